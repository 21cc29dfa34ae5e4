// Philox4x64-10 counter-based generator on the device.
//
// Written from the published definition: Salmon, Moraes, Dror, Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11, section 3.3. Each
// round takes the full 128-bit products of counter words 0 and 2 with two
// fixed odd multipliers, swaps the word pairs, and xors the high product
// halves with the other counter words and the round key; the key is bumped
// by two Weyl increments between rounds. Ten rounds.
//
// The verify step draws one block per (request b, position k): key
// (seed_b, 0), counter (b, k, 0, 0). Word 0 feeds the accept test at k and
// word 1 a draw at k, each as its top 24 bits times 2^-24 (exact in fp32 and
// fp64). The randomness consumed therefore does not depend on which path a
// request takes, which is the property the survey's "RNG consumed extra on
// the reject path" failure mode (section 23) asks for.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lvtv {

struct Philox4x64Out {
  uint64_t w[4];
};

__device__ __forceinline__ Philox4x64Out philox4x64_10(uint64_t c0, uint64_t c1,
                                                       uint64_t c2, uint64_t c3,
                                                       uint64_t k0, uint64_t k1) {
  constexpr uint64_t kMulA = 0xD2E7470EE14C6C93ull;
  constexpr uint64_t kMulB = 0xCA5A826395121157ull;
  constexpr uint64_t kBumpA = 0x9E3779B97F4A7C15ull;  // golden ratio
  constexpr uint64_t kBumpB = 0xBB67AE8584CAA73Bull;  // sqrt(3) - 1
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t hi_a = __umul64hi(kMulA, c0);
    const uint64_t lo_a = kMulA * c0;
    const uint64_t hi_b = __umul64hi(kMulB, c2);
    const uint64_t lo_b = kMulB * c2;
    const uint64_t n0 = hi_b ^ c1 ^ k0;
    const uint64_t n2 = hi_a ^ c3 ^ k1;
    c0 = n0;
    c1 = lo_b;
    c2 = n2;
    c3 = lo_a;
    k0 += kBumpA;
    k1 += kBumpB;
  }
  Philox4x64Out r;
  r.w[0] = c0;
  r.w[1] = c1;
  r.w[2] = c2;
  r.w[3] = c3;
  return r;
}

// (accept uniform, draw uniform) for request b, position k.
__device__ __forceinline__ void verify_uniforms(uint64_t seed, uint64_t b,
                                                uint64_t k, double& u_accept,
                                                double& u_draw) {
  const Philox4x64Out r = philox4x64_10(b, k, 0, 0, seed, 0);
  u_accept = (double)(r.w[0] >> 40) * 0x1p-24;
  u_draw = (double)(r.w[1] >> 40) * 0x1p-24;
}

}  // namespace lvtv
