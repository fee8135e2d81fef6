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
// Layout and mapping (gfx950): the summary of a (b, h) pair is stored
// d-quad-major ([D/4][CS][4] fp32), so for each d-quad consecutive lanes read
// consecutive 16-byte entries of consecutive sub-blocks.  L lanes (4, 2 or
// 1, by block size) split one sub-block's quads and add their partial dots
// with in-register lane exchanges: more, shorter non-temporal load streams
// per CU keep HBM busier than one long stream per lane.  Products and sums
// are in float64 (qbar is exact in float64), so the only rounding of
// consequence is the one-time fp32 rounding of the summary entries.  The
// block max is a DPP max over the nsub lanes of a block.  The kernel
// is bound by HBM bandwidth: 4 * D bytes per sub-block plus 4 bytes of logit.

#include "nosa_device.hpp"
#include "nosa_launch.hpp"

namespace nosa {

constexpr int kScoreThreads = 256;

typedef float f4 __attribute__((ext_vector_type(4)));

// L lanes share one sub-block, each taking D/4/L of its 16-byte d-quads
// (more, shorter load streams per CU than one lane per sub-block); a wave
// covers SPW = 64 / L sub-blocks.  Lane l: sub-block l % SPW, quad slice
// l / SPW.
template <int D, int L>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(int Hq, int Hkv, int bs, int ss, int max_blocks,
                                                              const uint16_t* __restrict__ q,
                                                              const float* __restrict__ k_summary,
                                                              const float* __restrict__ e_summary,
                                                              const int32_t* __restrict__ seq_lens,
                                                              float* __restrict__ score_q,
                                                              float* __restrict__ score_e) {
  constexpr int NQ = D / 4;        // 16-byte d-quads per summary row
  constexpr int QL = NQ / L;       // quads per lane
  constexpr int SPW = kWave / L;   // sub-blocks per wave
  constexpr int SPG = SPW * (kScoreThreads / kWave);  // per workgroup
  const int bh = blockIdx.y;
  const int b = bh / Hkv, h = bh % Hkv;
  const int G = Hq / Hkv;
  const int nsub = bs / ss;
  const int CS = max_blocks * nsub;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int s0 = blockIdx.x * SPG;
  const int s = s0 + w * SPW + lane % SPW;
  const int part = lane / SPW;
  const int T = min(max(seq_lens[b], 0), max_blocks * bs);
  const int nb = (T + bs - 1) / bs;
  if (s0 >= nb * nsub) return;  // whole workgroup past the last block

  // the group's query first (clamped, branch-free loads), then this lane's
  // slice of the summary row (index clamped into the row; results past the
  // end are masked later), so neither wait covers the other's loads
  const int dq = threadIdx.x < D ? threadIdx.x : 0;
  const uint16_t* qh = q + ((int64_t)b * Hq + (int64_t)h * G) * D + dq;
  uint16_t qraw[16];
#pragma unroll
  for (int g = 0; g < 16; ++g) qraw[g] = qh[(int64_t)min(g, G - 1) * D];
  const f4* p = reinterpret_cast<const f4*>(k_summary) + (int64_t)bh * NQ * CS + min(s, CS - 1) +
                (int64_t)(part * QL) * CS;
  f4 v[QL];
#pragma unroll
  for (int u = 0; u < QL; ++u) v[u] = __builtin_nontemporal_load(p + (int64_t)u * CS);
  const float ev = e_summary[(int64_t)bh * CS + min(s, CS - 1)];

  __shared__ double qbar[D];
  if (threadIdx.x < D) {
    double a = 0;
#pragma unroll
    for (int g = 0; g < 16; ++g) a += g < G ? (double)bf16_to_f32(qraw[g]) : 0.0;
    qbar[threadIdx.x] = a / (double)G;
  }
  const int i = s / nsub, j = s % nsub;
  const bool valid = i < nb && i * bs + j * ss < T;
  __syncthreads();

  double a0 = 0, a1 = 0, a2 = 0, a3 = 0;
#pragma unroll
  for (int u = 0; u < QL; ++u) {
    const int d = 4 * (part * QL + u);
    a0 = fma((double)v[u].x, qbar[d + 0], a0);
    a1 = fma((double)v[u].y, qbar[d + 1], a1);
    a2 = fma((double)v[u].z, qbar[d + 2], a2);
    a3 = fma((double)v[u].w, qbar[d + 3], a3);
  }
  double dot = (a0 + a1) + (a2 + a3);
  dot = xor_reduce<SPW, kWave>(dot, [](double x, double y) { return x + y; });  // the L slices
  if (!valid) dot = -INFINITY;
  float ek = valid ? ev : -INFINITY;
  // max over the nsub sub-blocks of each block: nsub <= SPW consecutive lanes
  dot = xor_reduce_below(dot, nsub, [](double x, double y) { return fmax(x, y); });
  ek = xor_reduce_below(ek, nsub, [](float x, float y) { return fmaxf(x, y); });
  if (valid && part == 0 && j == 0) {
    score_q[(int64_t)bh * max_blocks + i] = (float)(dot / sqrt((double)D));
    score_e[(int64_t)bh * max_blocks + i] = ek;
  }
}

hipError_t launch_score(const nosa_dims& d, const uint16_t* q, const float* k_summary,
                        const float* e_summary, const int32_t* seq_lens, float* score_q,
                        float* score_e, hipStream_t stream) {
  const int nsub = d.block_size / d.sub_block;
  const int CS = d.max_blocks * nsub;
  const int L = nsub <= 16 ? 4 : (nsub <= 32 ? 2 : 1);  // a block must fit one wave's sub-blocks
  const int per_wg = kScoreThreads / L;
  const dim3 grid((CS + per_wg - 1) / per_wg, d.batch * d.n_kv_heads);
#define NOSA_SCORE(DD, LL)                                                                                  \
  score_kernel<DD, LL><<<grid, kScoreThreads, 0, stream>>>(d.n_q_heads, d.n_kv_heads, d.block_size,         \
                                                           d.sub_block, d.max_blocks, q, k_summary, e_summary, \
                                                           seq_lens, score_q, score_e)
  if (d.head_dim == 128) {
    if (L == 4) NOSA_SCORE(128, 4);
    else if (L == 2) NOSA_SCORE(128, 2);
    else NOSA_SCORE(128, 1);
  } else {
    if (L == 4) NOSA_SCORE(64, 4);
    else if (L == 2) NOSA_SCORE(64, 2);
    else NOSA_SCORE(64, 1);
  }
#undef NOSA_SCORE
  return hipGetLastError();
}

}  // namespace nosa
