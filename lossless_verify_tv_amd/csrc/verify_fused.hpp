// Host-side interface of the single-read verify kernel (verify_fused.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lvtv {
namespace vf {

// Rows are cut into slices of 16384 tokens; the single-read kernel handles up
// to this many slices per row (V <= 524288). Larger V take the two-read
// pipeline.
constexpr int kMaxSlices = 32;

struct VerifyCall {
  const void* target;
  const void* draft;
  int dtype;
  bool vec_ok;
  const int32_t* tokens;
  const int32_t* kreq;
  const float* temp;
  const uint64_t* seed;
  int B, Kmax, V;
  int spin_limit;
  int32_t* acc_len;
  int32_t* out_tokens;
  float* alpha;
  int32_t* status;
};

bool applicable(int B, int Kmax, int V);
size_t workspace_bytes(int B, int Kmax, int V);
hipError_t run(const VerifyCall& c, void* workspace, hipStream_t stream);

}  // namespace vf
}  // namespace lvtv
