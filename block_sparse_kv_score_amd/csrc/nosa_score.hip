// Block scoring for selection.
//
// NOSA summary (gist.science 2510.13602), Methodology 1: the query-aware
// part of dual selection scores blocks with the query; the query-agnostic
// part scores them with the eviction head's per-token logits; both scores
// are pooled in two stages -- a mean inside each sub-block, then a max over
// the block -- and ED-DMA keeps the exponent out of selection, so raw logits
// are pooled.
//
// The query-aware token score is the group mean of q_g . k / sqrt(D).  By
// linearity, the sub-block mean of that score equals qbar . kbar / sqrt(D)
// with qbar the mean of the group's queries and kbar the sub-block mean key,
// so the kernel streams the fp32 sub-block summaries instead of every key.
//
// Layout and mapping (gfx950): one lane per sub-block; the summary of a
// (b, h) pair is stored d-quad-major ([D/4][CS][4] fp32), so for each d-quad
// a wave reads 64 consecutive 16-byte entries (1 KiB, fully coalesced) and
// no cross-lane reduction is needed for the dot product.  Products and sums
// are in float64 (qbar is exact in float64), so the only rounding of
// consequence is the one-time fp32 rounding of the summary entries.  The
// block max is a DPP/shuffle max over the nsub lanes of a block.  The kernel
// is bound by HBM bandwidth: 4 * D bytes per sub-block plus 4 bytes of logit.

#include "nosa_launch.hpp"

namespace nosa {

constexpr int kScoreThreads = 256;

template <int D>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(int Hq, int Hkv, int bs, int ss, int max_blocks,
                                                              const uint16_t* __restrict__ q,
                                                              const float* __restrict__ k_summary,
                                                              const float* __restrict__ e_summary,
                                                              const int32_t* __restrict__ seq_lens,
                                                              float* __restrict__ score_q,
                                                              float* __restrict__ score_e) {
  constexpr int NQ = D / 4;
  const int bh = blockIdx.y;
  const int b = bh / Hkv, h = bh % Hkv;
  const int G = Hq / Hkv;
  const int nsub = bs / ss;
  const int CS = max_blocks * nsub;
  const int T = min(max(seq_lens[b], 0), max_blocks * bs);
  const int nb = (T + bs - 1) / bs;
  const int s0 = blockIdx.x * kScoreThreads;
  if (s0 >= nb * nsub) return;  // whole workgroup past the last block

  const int s = s0 + threadIdx.x;
  const int i = s / nsub, j = s % nsub;
  const bool valid = i < nb && i * bs + j * ss < T;

  // issue every load of the row first: D/4 independent 16-byte loads per
  // lane (each a 1 KiB contiguous run per wave) keep the HBM queues full
  // while the group-mean query is formed
  typedef float f4 __attribute__((ext_vector_type(4)));
  f4 v[NQ];
  float ev = -INFINITY;
  if (valid) {
    const f4* kp = reinterpret_cast<const f4*>(k_summary) + (int64_t)bh * NQ * CS + s;
#pragma unroll
    for (int u = 0; u < NQ; ++u) v[u] = __builtin_nontemporal_load(kp + (int64_t)u * CS);
    ev = e_summary[(int64_t)bh * CS + s];
  }

  __shared__ double qbar[D];
  for (int d = threadIdx.x; d < D; d += kScoreThreads) {
    const uint16_t* qh = q + ((int64_t)b * Hq + (int64_t)h * G) * D + d;
    double a = 0;
    for (int g = 0; g < G; ++g) a += (double)bf16_to_f32(qh[(int64_t)g * D]);
    qbar[d] = a / (double)G;
  }
  __syncthreads();

  double dot = -INFINITY;
  if (valid) {
    double a0 = 0, a1 = 0, a2 = 0, a3 = 0;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      a0 = fma((double)v[u].x, qbar[4 * u + 0], a0);
      a1 = fma((double)v[u].y, qbar[4 * u + 1], a1);
      a2 = fma((double)v[u].z, qbar[4 * u + 2], a2);
      a3 = fma((double)v[u].w, qbar[4 * u + 3], a3);
    }
    dot = (a0 + a1) + (a2 + a3);
  }
  // max over the nsub lanes of each block (nsub is a power of two <= 64 and
  // kScoreThreads is a multiple of 64, so a block never straddles a wave)
  for (int off = 1; off < nsub; off <<= 1) {
    dot = fmax(dot, __shfl_xor(dot, off, kWave));
    ev = fmaxf(ev, __shfl_xor(ev, off, kWave));
  }
  if (valid && j == 0) {
    score_q[(int64_t)bh * max_blocks + i] = (float)(dot / sqrt((double)D));
    score_e[(int64_t)bh * max_blocks + i] = ev;
  }
}

hipError_t launch_score(const nosa_dims& d, const uint16_t* q, const float* k_summary,
                        const float* e_summary, const int32_t* seq_lens, float* score_q,
                        float* score_e, hipStream_t stream) {
  const int CS = d.max_blocks * (d.block_size / d.sub_block);
  const dim3 grid((CS + kScoreThreads - 1) / kScoreThreads, d.batch * d.n_kv_heads);
  if (d.head_dim == 128)
    score_kernel<128><<<grid, kScoreThreads, 0, stream>>>(d.n_q_heads, d.n_kv_heads, d.block_size,
                                                          d.sub_block, d.max_blocks, q, k_summary,
                                                          e_summary, seq_lens, score_q, score_e);
  else
    score_kernel<64><<<grid, kScoreThreads, 0, stream>>>(d.n_q_heads, d.n_kv_heads, d.block_size,
                                                         d.sub_block, d.max_blocks, q, k_summary,
                                                         e_summary, seq_lens, score_q, score_e);
  return hipGetLastError();
}

}  // namespace nosa
