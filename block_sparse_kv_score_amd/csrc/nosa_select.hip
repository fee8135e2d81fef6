// Dual selection and the block-swap set differences.
//
// NOSA summary (gist.science 2510.13602), Methodology 1: selection is split
// into a query-aware part (recall, possibly far-away blocks) and a
// query-agnostic eviction part that follows a strict policy -- whatever it
// leaves out once it never takes back; with a fixed budget k_e for that part
// most blocks chosen at step t were chosen at t-1 (locality at least
// k_e / k).  Methodology 2 (NOSI): set differences between consecutive block
// sets drive block swapping.
//
// Readings: the two parts are disjoint (the query part picks among blocks
// the eviction part did not take), the never-return rule binds the eviction
// part only, ties go to the lower block index, and a newly created block
// starts as an eviction candidate.
//
// One workgroup per (b, h).  Top-k is a most-significant-digit radix select
// over order-preserving 32-bit keys of the fp32 scores with 4-bit digits:
// each pass counts the 16 digit values with wave ballots (no LDS atomics,
// which would serialise on the few crowded bins), sums the four waves'
// counts through LDS and picks the bin holding the k-th key; it stops as
// soon as that bin is taken whole.  Exact key ties go to the lowest index.
// Outputs are compacted in index order with wave ballots, so they come out
// ascending without a sort.

#include "nosa_launch.hpp"

namespace nosa {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kMaxBlocks = 8192;

// flag bits per block in LDS
constexpr uint8_t F_EVICTED = 1;  // evicted before or during this call
constexpr uint8_t F_IN_E = 2;     // in Gamma_e
constexpr uint8_t F_IN_Q = 4;     // in Gamma_q

struct SelShared {
  uint32_t key[kMaxBlocks];
  uint8_t flag[kMaxBlocks];
  int32_t cnt[kSelWaves][16];
  int32_t wave_tot[kSelWaves];
  int32_t bcast[4];
};

// Exclusive count of `pred` over the workgroup in thread order, plus the
// total.  Every thread must call it.
__device__ __forceinline__ int block_count_excl(bool pred, int& total, SelShared& sh) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const uint64_t m = __ballot(pred);
  const int below = lanes_below(m);
  if (lane == 0) sh.wave_tot[w] = __popcll(m);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < kSelWaves; ++k) {
    const int c = sh.wave_tot[k];
    before += k < w ? c : 0;
    total += c;
  }
  __syncthreads();
  return before + below;
}

// Marks with `mark` the k best of the candidates (flag & cmask) == cval
// under (key desc, index asc).  Requires 0 < k < number of candidates.
__device__ void radix_top_k(int n, int k, uint8_t cmask, uint8_t cval, uint8_t mark, SelShared& sh) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  uint32_t prefix = 0, pmask = 0;
  int rem = k;   // still to take among keys matching the prefix
  int n_eq = 0;  // candidates matching the prefix
  for (int shift = 28; shift >= 0; shift -= 4) {
    int cnt[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) cnt[d] = 0;
    for (int base = 0; base < n; base += kSelThreads) {
      const int i = base + threadIdx.x;
      const uint32_t key = i < n ? sh.key[i] : 0u;
      const bool in = i < n && (sh.flag[i] & cmask) == cval && (key & pmask) == prefix;
      const uint32_t dg = (key >> shift) & 15u;
#pragma unroll
      for (int d = 0; d < 16; ++d) cnt[d] += __popcll(__ballot(in && dg == (uint32_t)d));
    }
    if (lane == 0) {
#pragma unroll
      for (int d = 0; d < 16; ++d) sh.cnt[w][d] = cnt[d];
    }
    __syncthreads();
    // lanes 0..15 of every wave take one digit each: total over the waves,
    // suffix sum from the top digit, and the lane whose range holds the
    // rem-th key names the digit (every wave computes the same answer)
    int c = 0;
    if (lane < 16) {
#pragma unroll
      for (int ww = 0; ww < kSelWaves; ++ww) c += sh.cnt[ww][lane];
    }
    int suf = c;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int t = __shfl_down(suf, off, kWave);
      if (lane + off < 16) suf += t;
    }
    const uint64_t hit = __ballot(lane < 16 && suf >= rem && suf - c < rem);
    const int digit = __ffsll((unsigned long long)hit) - 1;
    const int above = __shfl(suf - c, digit, kWave);
    const int bin = __shfl(c, digit, kWave);
    rem -= above;
    n_eq = bin;
    prefix |= (uint32_t)digit << shift;
    pmask |= 15u << shift;
    __syncthreads();
    if (rem == n_eq) break;  // the whole bin is taken: prefix is the threshold
  }
  const uint32_t thr = prefix;
  if (rem == n_eq) {
    for (int i = threadIdx.x; i < n; i += kSelThreads)
      if ((sh.flag[i] & cmask) == cval && sh.key[i] >= thr) sh.flag[i] |= mark;
    __syncthreads();
    return;
  }
  // exact key ties: take the rem lowest indices among keys equal to thr
  int carry = 0;
  for (int base = 0; base < n; base += kSelThreads) {
    const int i = base + threadIdx.x;
    const bool cand = i < n && (sh.flag[i] & cmask) == cval;
    const uint32_t key = cand ? sh.key[i] : 0u;
    const bool eq = cand && key == thr;
    int total;
    const int rank = carry + block_count_excl(eq, total, sh);
    if (cand && (key > thr || (eq && rank < rem))) sh.flag[i] |= mark;
    carry += total;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(int Hkv, int bs, int max_blocks,
                                                             const float* __restrict__ score_q,
                                                             const float* __restrict__ score_e,
                                                             const int32_t* __restrict__ seq_lens,
                                                             int k_e, int k_q,
                                                             uint32_t* __restrict__ evicted,
                                                             int32_t* __restrict__ sel, int sel_cap,
                                                             int32_t* __restrict__ sel_count) {
  __shared__ SelShared sh;
  const int bh = blockIdx.x;
  const int b = bh / Hkv;
  const int T = min(max(seq_lens[b], 0), max_blocks * bs);
  const int nb = (T + bs - 1) / bs;
  const int words = (max_blocks + 31) / 32;
  uint32_t* ev = evicted + (int64_t)bh * words;
  const float* se = score_e + (int64_t)bh * max_blocks;
  const float* sq = score_q + (int64_t)bh * max_blocks;

  // --- eviction part ------------------------------------------------------
  for (int i = threadIdx.x; i < nb; i += kSelThreads) {
    sh.flag[i] = ((ev[i >> 5] >> (i & 31)) & 1u) ? F_EVICTED : 0;
    sh.key[i] = order_key(se[i]);
  }
  __syncthreads();
  int n_cand = 0;
  for (int base = 0; base < nb; base += kSelThreads) {
    const int i = base + threadIdx.x;
    int total;
    block_count_excl(i < nb && !(sh.flag[i] & F_EVICTED), total, sh);
    n_cand += total;
  }
  const int n_e = min(k_e, n_cand);
  if (n_e == n_cand) {
    for (int i = threadIdx.x; i < nb; i += kSelThreads)
      if (!(sh.flag[i] & F_EVICTED)) sh.flag[i] |= F_IN_E;
  } else if (n_e > 0) {
    radix_top_k(nb, n_e, F_EVICTED, 0, F_IN_E, sh);
  }
  __syncthreads();
  // every candidate left out is evicted for good
  for (int i = threadIdx.x; i < nb; i += kSelThreads)
    if (!(sh.flag[i] & (F_EVICTED | F_IN_E))) sh.flag[i] |= F_EVICTED;
  __syncthreads();

  // --- query part ---------------------------------------------------------
  for (int i = threadIdx.x; i < nb; i += kSelThreads) sh.key[i] = order_key(sq[i]);
  __syncthreads();
  const int rest = nb - n_e;
  const int n_q = min(k_q, rest);
  if (n_q == rest) {
    for (int i = threadIdx.x; i < nb; i += kSelThreads)
      if (!(sh.flag[i] & F_IN_E)) sh.flag[i] |= F_IN_Q;
  } else if (n_q > 0) {
    radix_top_k(nb, n_q, F_IN_E, 0, F_IN_Q, sh);
  }
  __syncthreads();

  // --- outputs: ascending union, evicted bitmap ----------------------------
  int carry = 0;
  int32_t* out = sel + (int64_t)bh * sel_cap;
  for (int base = 0; base < nb; base += kSelThreads) {
    const int i = base + threadIdx.x;
    const bool pick = i < nb && (sh.flag[i] & (F_IN_E | F_IN_Q));
    int total;
    const int pos = carry + block_count_excl(pick, total, sh);
    if (pick && pos < sel_cap) out[pos] = i;
    carry += total;
  }
  if (threadIdx.x == 0) sel_count[bh] = min(carry, sel_cap);
  for (int w = threadIdx.x; w < (nb + 31) / 32; w += kSelThreads) {
    uint32_t bits = 0;
    for (int k = 0; k < 32; ++k) {
      const int i = w * 32 + k;
      if (i < nb && (sh.flag[i] & F_EVICTED)) bits |= 1u << k;
    }
    ev[w] |= bits;
  }
}

// One wave per (b, h); membership through an LDS bitmap, order-preserving
// compaction through ballots.
__global__ __launch_bounds__(kWave) void swap_diff_kernel(int max_blocks, int cap,
                                                          const int32_t* __restrict__ prev,
                                                          const int32_t* __restrict__ prev_count,
                                                          const int32_t* __restrict__ cur,
                                                          const int32_t* __restrict__ cur_count,
                                                          int32_t* __restrict__ load,
                                                          int32_t* __restrict__ load_count,
                                                          int32_t* __restrict__ evict,
                                                          int32_t* __restrict__ evict_count) {
  __shared__ uint32_t bm[kMaxBlocks / 32];
  const int bh = blockIdx.x;
  const int lane = threadIdx.x;
  const int np = min(max(prev_count[bh], 0), cap);
  const int nc = min(max(cur_count[bh], 0), cap);
  const int32_t* p = prev + (int64_t)bh * cap;
  const int32_t* c = cur + (int64_t)bh * cap;

  // pass 0: load = cur \ prev;  pass 1: evict = prev \ cur
  for (int pass = 0; pass < 2; ++pass) {
    const int32_t* mark_list = pass == 0 ? p : c;
    const int n_mark = pass == 0 ? np : nc;
    const int32_t* test_list = pass == 0 ? c : p;
    const int n_test = pass == 0 ? nc : np;
    int32_t* out = (pass == 0 ? load : evict) + (int64_t)bh * cap;
    for (int w = lane; w < kMaxBlocks / 32; w += kWave) bm[w] = 0;
    wave_lds_sync();
    for (int k = lane; k < n_mark; k += kWave) {
      const int x = mark_list[k];
      if (x >= 0 && x < max_blocks) atomicOr(&bm[x >> 5], 1u << (x & 31));
    }
    wave_lds_sync();
    int n_out = 0;
    for (int base = 0; base < n_test; base += kWave) {
      const int k = base + lane;
      const int x = k < n_test ? test_list[k] : -1;
      const bool keep = x >= 0 && x < max_blocks && !((bm[x >> 5] >> (x & 31)) & 1u);
      const uint64_t m = __ballot(keep);
      if (keep) out[n_out + lanes_below(m)] = x;
      n_out += __popcll(m);
    }
    if (lane == 0) (pass == 0 ? load_count : evict_count)[bh] = n_out;
    wave_lds_sync();
  }
}

hipError_t launch_select(const nosa_dims& d, const float* score_q, const float* score_e,
                         const int32_t* seq_lens, int32_t k_e, int32_t k_q, uint32_t* evicted,
                         int32_t* sel, int32_t sel_cap, int32_t* sel_count, hipStream_t stream) {
  select_kernel<<<d.batch * d.n_kv_heads, kSelThreads, 0, stream>>>(
      d.n_kv_heads, d.block_size, d.max_blocks, score_q, score_e, seq_lens, k_e, k_q, evicted, sel,
      sel_cap, sel_count);
  return hipGetLastError();
}

hipError_t launch_swap_diff(const nosa_dims& d, int32_t cap, const int32_t* prev,
                            const int32_t* prev_count, const int32_t* cur, const int32_t* cur_count,
                            int32_t* load, int32_t* load_count, int32_t* evict,
                            int32_t* evict_count, hipStream_t stream) {
  swap_diff_kernel<<<d.batch * d.n_kv_heads, kWave, 0, stream>>>(
      d.max_blocks, cap, prev, prev_count, cur, cur_count, load, load_count, evict, evict_count);
  return hipGetLastError();
}

}  // namespace nosa
