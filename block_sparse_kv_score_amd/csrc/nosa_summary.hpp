// Sub-block sums for the summaries that block scoring pools over (NOSA
// summary (gist.science 2510.13602), Methodology 1, block-wise
// implementation: the mean inside each sub-block is the first pooling
// stage).
//
// Sums over a sub-block's present tokens [lo, hi) (page-relative) are taken
// in float64 in ascending token order.  Loads go out in batches of BATCH
// tokens (clamped, branch-free); padding slots add +0.0, which leaves a
// float64 sum unchanged, so every caller produces identical sums for
// identical tokens whatever its batch size.
#pragma once

#include "nosa_device.hpp"

namespace nosa {

constexpr int kSumBatch = 16;

// quad u = dims 4u..4u+3 of a K page [D/8][bs][8] = half (u & 1) of octet u >> 1
template <int D, int BATCH = kSumBatch>
__device__ __forceinline__ void sum_key_quad(const uint16_t* kpage, int bs, int u, int lo, int hi,
                                             double& a0, double& a1, double& a2, double& a3) {
  const uint2* base = reinterpret_cast<const uint2*>(kpage) + ((u >> 1) * bs) * 2 + (u & 1);
  for (int t0 = lo; t0 < hi; t0 += BATCH) {
    uint2 v[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) v[j] = base[min(t0 + j, hi - 1) * 2];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const bool in = t0 + j < hi;
      a0 += in ? (double)bf16_lo(v[j].x) : 0.0;
      a1 += in ? (double)bf16_hi(v[j].x) : 0.0;
      a2 += in ? (double)bf16_lo(v[j].y) : 0.0;
      a3 += in ? (double)bf16_hi(v[j].y) : 0.0;
    }
  }
}

template <int BATCH = kSumBatch>
__device__ __forceinline__ double sum_logits(const float* ep, int lo, int hi) {
  double a = 0;
  for (int t0 = lo; t0 < hi; t0 += BATCH) {
    float v[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) v[j] = ep[min(t0 + j, hi - 1)];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) a += t0 + j < hi ? (double)v[j] : 0.0;
  }
  return a;
}

}  // namespace nosa
