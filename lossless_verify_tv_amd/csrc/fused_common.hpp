// Cross-workgroup exchange for the single-read kernels (gfx950).
//
// A row of V = 1.5e5 bf16 logits is spread over several workgroups, each
// holding its slice in registers. They swap a few numbers (slice softmax
// statistics, partial sums) through a workspace of 64-bit tagged words: the
// high half is a tag naming the call, the low half the payload, written and
// read with single relaxed agent-scope atomic accesses. A reader knows a
// word is fresh when its tag is the current one, so no fences, no resets and
// no ordering between different words are needed.
//
// Calls are told apart by an epoch counter in the workspace control block;
// the tag is derived from it and is never 0, so a zero-filled workspace
// holds no fresh word. The call's last launch advances the epoch, so the
// next call's tag differs and nothing a call leaves behind is ever taken for
// fresh. The workspace must therefore be zero-filled once before its first
// use (lvtv_workspace_reset).
//
// Every wait is bounded: a workgroup that polls a word for `spin_limit`
// rounds without seeing it gives up, and the missing values are recomputed
// from the inputs with the same functions (same element order, same
// reduction tree) their producers use, so the result is bit-identical either
// way and no schedule of workgroups can deadlock.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace lvtv {

struct FusedCtl {
  uint32_t epoch;  // bumped once per completed call
  uint32_t unused;
  uint32_t pad[62];
};
static_assert(sizeof(FusedCtl) == 256, "control block is one 256-byte line");

// Every workspace starts with a region of fixed layout, whatever the call's
// shapes: the control block, then room for one 32-bit counter per unit of
// work (a request or a branch; the current kernels keep none there). The
// shape-dependent arrays (tagged words, partial sums) come after it.
constexpr int kMaxUnits = 65536;
constexpr size_t kReservedBytes = sizeof(FusedCtl) + sizeof(uint32_t) * size_t(kMaxUnits);
static_assert(kReservedBytes % 256 == 0, "reserved region keeps 256-byte alignment");

__host__ __device__ inline FusedCtl* workspace_ctl(void* ws) { return static_cast<FusedCtl*>(ws); }
__host__ __device__ inline uint32_t* workspace_counters(void* ws) {
  return reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + sizeof(FusedCtl));
}

__device__ __forceinline__ uint32_t tag_from_epoch(uint32_t epoch) {
  return ((epoch & 0x7fffffffu) << 1) | 1u;
}

__device__ __forceinline__ uint32_t read_epoch(FusedCtl* ctl) {
  return __hip_atomic_load(&ctl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void tag_store(uint64_t* p, uint32_t tag, uint32_t bits) {
  __hip_atomic_store(p, (uint64_t(tag) << 32) | uint64_t(bits), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t tag_load(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Nontemporal 16-byte vector loads/stores: streamed data is read once.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// The same from an address that is only 2-byte aligned. Code objects for
// this target run in unaligned access mode (the compiler emits one 16-byte
// load for such a type), so this stays a single vector load; the caller makes
// sure that all 16 bytes lie inside the row.
typedef u32x4 u32x4_u __attribute__((aligned(2)));

__device__ __forceinline__ u32x4 ld_nt16_u(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_u*>(p));
}

__device__ __forceinline__ u32x4 ld16_u(const void* p) {
  return *reinterpret_cast<const u32x4_u*>(p);
}

__device__ __forceinline__ void st_nt16_u(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_u*>(p));
}

// A group's tokens moved down by s places (token j takes token j + s), the
// top places taking `fill`: s >= 8 leaves only fill. bf16 tokens, two a word.
__device__ __forceinline__ u32x4 shift_bf16(u32x4 w, uint32_t s, uint32_t fill) {
  if (s & 4) w = u32x4{w[2], w[3], fill, fill};
  if (s & 2) w = u32x4{w[1], w[2], w[3], fill};
  if (s & 1)
    w = u32x4{__builtin_amdgcn_alignbyte(w[1], w[0], 2), __builtin_amdgcn_alignbyte(w[2], w[1], 2),
              __builtin_amdgcn_alignbyte(w[3], w[2], 2), __builtin_amdgcn_alignbyte(fill, w[3], 2)};
  return s >= 8 ? u32x4{fill, fill, fill, fill} : w;
}

// The same for 8 fp32 tokens, one a word, in a (tokens 0-3) and b (4-7).
__device__ __forceinline__ void shift_f32(u32x4& a, u32x4& b, uint32_t s, uint32_t fill) {
  const u32x4 f = u32x4{fill, fill, fill, fill};
  if (s & 4) {
    a = b;
    b = f;
  }
  if (s & 2) {
    a = u32x4{a[2], a[3], b[0], b[1]};
    b = u32x4{b[2], b[3], fill, fill};
  }
  if (s & 1) {
    a = u32x4{a[1], a[2], a[3], b[0]};
    b = u32x4{b[1], b[2], b[3], fill};
  }
  if (s >= 8) a = b = f;
}

__device__ __forceinline__ void st_nt16(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

}  // namespace lvtv
