// Library-level entry points of the C ABI (version, error strings,
// workspace reset).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/lvtv.h"

namespace {

// Zero fill with vector stores (a plain kernel, so the reset can sit inside
// a captured graph).
__global__ void zero_fill(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

extern "C" int lvtv_workspace_reset(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return LVTV_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return LVTV_ERR_WORKSPACE;
  const size_t n16 = workspace_bytes / 16;
  const size_t ntail = workspace_bytes - n16 * 16;
  if (workspace_bytes == 0) return LVTV_OK;
  size_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_fill, dim3(unsigned(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(workspace), n16,
                     static_cast<unsigned char*>(workspace) + n16 * 16, ntail);
  return hipGetLastError() == hipSuccess ? LVTV_OK : LVTV_ERR_LAUNCH;
}

extern "C" int lvtv_version(void) { return 1; }

extern "C" const char* lvtv_strerror(int code) {
  switch (code) {
    case LVTV_OK: return "ok";
    case LVTV_ERR_NULL: return "a required pointer is NULL";
    case LVTV_ERR_SHAPE: return "a size is outside the supported range";
    case LVTV_ERR_DTYPE: return "unknown dtype";
    case LVTV_ERR_WORKSPACE: return "workspace is NULL, misaligned or smaller than required";
    case LVTV_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case LVTV_ERR_OBJECTIVE: return "unknown loss objective";
    case LVTV_ERR_TEMPERATURE: return "temperature not finite and > 0 (or 1/T overflows)";
    case LVTV_ERR_OPTION: return "unknown debug option";
    case LVTV_ERR_SCRATCH: return "sizes need more than the no-allocation scratch holds";
    default: return "unknown error code";
  }
}
