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
// over order-preserving 32-bit keys of the fp32 scores (four 8-bit passes,
// each an LDS histogram plus a workgroup suffix scan), followed by a
// lowest-index-first pick among blocks whose key equals the threshold.
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
  uint32_t hist[256];
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

// Inclusive scan of one int per thread, in thread order.
__device__ __forceinline__ int block_scan_incl(int v, SelShared& sh) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  if (lane == kWave - 1) sh.wave_tot[w] = v;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int k = 0; k < kSelWaves; ++k) before += k < w ? sh.wave_tot[k] : 0;
  __syncthreads();
  return v + before;
}

// Marks with `mark` the k best of the candidates (flag & cmask) == cval
// under (key desc, index asc).  Requires 0 < k < number of candidates.
__device__ void radix_top_k(int n, int k, uint8_t cmask, uint8_t cval, uint8_t mark, SelShared& sh) {
  uint32_t prefix = 0, pmask = 0;
  int rem = k;       // still to take among keys matching the prefix
  int n_eq = 0;      // candidates whose key equals the final threshold
  for (int shift = 24; shift >= 0; shift -= 8) {
    sh.hist[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kSelThreads) {
      const uint32_t key = sh.key[i];
      if ((sh.flag[i] & cmask) == cval && (key & pmask) == prefix)
        atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // suffix counts: thread t owns digit 255 - t
    const int cnt = (int)sh.hist[255 - threadIdx.x];
    const int cum = block_scan_incl(cnt, sh);  // #keys with digit >= 255 - t
    if (cum >= rem && cum - cnt < rem) {
      sh.bcast[0] = 255 - threadIdx.x;
      sh.bcast[1] = cum - cnt;
      sh.bcast[2] = cnt;
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)sh.bcast[0];
    rem -= sh.bcast[1];
    n_eq = sh.bcast[2];
    prefix |= digit << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t thr = prefix;
  if (rem == n_eq) {
    for (int i = threadIdx.x; i < n; i += kSelThreads)
      if ((sh.flag[i] & cmask) == cval && sh.key[i] >= thr) sh.flag[i] |= mark;
    __syncthreads();
    return;
  }
  // take the rem lowest indices among the keys equal to thr
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
