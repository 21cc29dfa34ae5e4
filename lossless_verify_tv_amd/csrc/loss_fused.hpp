// Host-side interface of the single-read loss kernel (loss_fused.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lvtv {
namespace lf {

// A row is held in registers as kMaxGroups groups of 8 tokens per thread of
// a 1024-thread workgroup: V up to 155648 (larger V take the multi-pass
// pipeline).
constexpr int kMaxGroups = 19;
constexpr int kMaxV = kMaxGroups * 1024 * 8;

struct LossCall {
  const uint16_t* z;
  const float* p;         // target probabilities, or null with ...
  const uint16_t* t;      // ... target logits (temperature on both rows)
  float c;                // exponent scale fl32(log2(e) fl32(1/T)) (log2(e) at T = 1)
  double inv_t;           // chain factor fl32(1/T) of the gradient
  int N, W, V;
  int objective;  // LVTV_OBJ_E2E_TV or LVTV_OBJ_STEP_TV
  bool vec_ok;
  bool reread;            // CE / KL: every row's dz from a second read of p (debug)
  int spin_limit;
  float* loss;
  float* alpha;
  uint16_t* dz;
  float* dz32;            // debug: fp32 gradient before rounding, or null
};

bool applicable(int N, int W, int V);
// Whether the single-read kernel takes a logits target.
bool logits_supported();
// Whether the single-read kernel takes CE and KL (probability target only).
bool xent_supported(bool logits);
size_t workspace_bytes(int N, int W, int V);
hipError_t run(const LossCall& c, void* workspace, hipStream_t stream);

}  // namespace lf
}  // namespace lvtv
