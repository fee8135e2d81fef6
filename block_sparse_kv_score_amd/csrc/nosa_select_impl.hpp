// Dual selection and the swap lists for one (b, h) pair, as a workgroup
// device function, shared by the selection kernel and the decode kernel's
// select variant.
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
// NT threads per (b, h) (256: the four-wave form; 1024 for the widest
// tables); each keeps its blocks' keys in registers (block i = r * NT +
// thread).  Top-k is a most-significant-digit radix
// select over order-preserving 32-bit keys of the fp32 scores (see
// radix_top_k); exact key ties go to the lowest index.  Outputs are
// compacted in index order with wave ballots, so they come out ascending
// without a sort, and the eviction bitmap words are rebuilt from ballots.
// (A one-wave form with 16 elements per lane, free of workgroup barriers,
// measured slower for 516 blocks.)
#pragma once

#include <type_traits>

#include "nosa_device.hpp"

namespace nosa {

constexpr int kSelThreads = 256;                // the four-wave form
constexpr int kMaxBlocks = 8192;
constexpr int kDigitWaves = 256 / kWave;         // waves that scan the 256 digit bins

// Per-workgroup scratch in LDS; small slots are double-buffered by phase so
// one barrier per exchange suffices.
template <int NT>
struct SelSharedT {
  static constexpr int NW = NT / kWave;
  uint32_t hist[NW][256];  // per-wave digit histograms
  int32_t tot[2][NW];
  int32_t bc[2][4];
  uint32_t mm[2][NW][2];
  int32_t pos[32][NW];
  // fused swap lists: membership bitmaps and per-wave counts
  uint32_t pick_bm[kMaxBlocks / 32];
  uint32_t prev_bm[kMaxBlocks / 32];
  int32_t pos_load[32][NW];
  int32_t pos_evict[32][NW];
};
using SelShared = SelSharedT<kSelThreads>;

// Workgroup sum of one int per wave (the same value in every lane); one
// barrier.
template <int NT>
__device__ __forceinline__ int block_sum(int v, int& phase, SelSharedT<NT>& sh) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int ph = phase++ & 1;
  if (lane == 0) sh.tot[ph][w] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) t += sh.tot[ph][k];
  return t;
}

// Element r of this thread is block i = r * kSelThreads + threadIdx.x; the
// thread's R elements live in registers (keys) and bit masks (bit r).
// Marks in `out` the k best of the elements in `cand` under (key desc,
// index asc).  Requires 0 < k < number of candidates.
//
// Radix select over 8-bit digits.  The first digit starts at the highest
// bit where the candidates' smallest and largest keys differ (the bits above
// are common to all of them), so no pass is spent on a shared exponent.
// Digits are counted in per-wave LDS histograms; a workgroup scan over the
// 256 bins finds the bin holding the k-th key; the select stops as soon as
// that bin is taken whole.
template <int R, int NT>
__device__ __forceinline__ void radix_top_k(const uint32_t (&key)[R], uint32_t cand, int k, uint32_t& out, int& phase,
                            SelSharedT<NT>& sh) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  // range of the candidate keys
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if ((cand >> r) & 1u) {
      kmin = min(kmin, key[r]);
      kmax = max(kmax, key[r]);
    }
  kmin = xor_reduce<1, kWave>(kmin, [](uint32_t a, uint32_t b) { return min(a, b); });
  kmax = xor_reduce<1, kWave>(kmax, [](uint32_t a, uint32_t b) { return max(a, b); });
  {
    const int ph = phase++ & 1;
    if (lane == 0) {
      sh.mm[ph][w][0] = kmin;
      sh.mm[ph][w][1] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      kmin = min(kmin, sh.mm[ph][ww][0]);
      kmax = max(kmax, sh.mm[ph][ww][1]);
    }
  }
  int hi = kmin == kmax ? 0 : 32 - __clz(kmin ^ kmax);  // bits [hi, 32) are shared
  uint32_t prefix = hi >= 32 ? 0u : kmin & ~((1u << hi) - 1u);
  uint32_t pmask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
  int rem = k, n_eq = 0;
  bool done = false;
  while (hi > 0 && !done) {
    const int lo = hi > 8 ? hi - 8 : 0;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    // per-wave histogram of this digit among the keys matching the prefix
#pragma unroll
    for (int j = 0; j < 4; ++j) sh.hist[w][lane + 64 * j] = 0u;
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (((cand >> r) & 1u) && (key[r] & pmask) == prefix) atomicAdd(&sh.hist[w][(key[r] >> lo) & dmask], 1u);
    __syncthreads();
    const int ph = phase++ & 1;
    // thread t < 256 owns digit 255 - t: inclusive scan gives the count of
    // keys with a digit >= 255 - t (the other threads of a wider workgroup
    // count nothing)
    const bool owner = NT == 256 || (int)threadIdx.x < 256;
    const int dg = owner ? 255 - (int)threadIdx.x : 0;
    int c = 0;
    if (owner) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) c += (int)sh.hist[ww][dg];
    }
    int cum = wave_scan_incl(c);
    if (lane == kWave - 1 && w < kDigitWaves) sh.tot[ph][w] = cum;
    __syncthreads();
#pragma unroll
    for (int ww = 0; ww < kDigitWaves; ++ww) cum += ww < w ? sh.tot[ph][ww] : 0;
    if (c > 0 && cum >= rem && cum - c < rem) {
      sh.bc[ph][0] = dg;
      sh.bc[ph][1] = cum - c;
      sh.bc[ph][2] = c;
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)sh.bc[ph][0];
    rem -= sh.bc[ph][1];
    n_eq = sh.bc[ph][2];
    prefix |= digit << lo;
    pmask |= dmask << lo;
    hi = lo;
    done = rem == n_eq;  // the whole bin is taken: prefix is the threshold
  }
  if (rem == n_eq) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (((cand >> r) & 1u) && (key[r] & pmask) >= prefix) out |= 1u << r;
    return;
  }
  // exact key ties at the threshold: the rem lowest block indices win
  uint64_t eqm[R];
#pragma unroll
  for (int r = 0; r < R; ++r) eqm[r] = __ballot(((cand >> r) & 1u) && key[r] == prefix);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) sh.pos[r][w] = __popcll(eqm[r]);
  }
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int rank = before + lanes_below(eqm[r]);
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const int c = sh.pos[r][ww];
      rank += ww < w ? c : 0;
      before += c;
    }
    if ((cand >> r) & 1u) {
      if (key[r] > prefix || (key[r] == prefix && rank < rem)) out |= 1u << r;
    }
  }
  __syncthreads();  // sh.pos is reused by the caller
}

struct SwapArgs {
  const int32_t* prev;
  const int32_t* prev_count;
  int32_t* load;
  int32_t* load_count;
  int32_t* evict;
  int32_t* evict_count;
};

// Selection of pair bh over its first T tokens (nb = ceil(T / bs) blocks),
// called by all NT threads of a workgroup; returns the selection size (the
// same value in every thread).  R elements per thread cover max_blocks
// (R * NT >= max_blocks).
//   sq_row, se_row: the pair's max_blocks query-aware and eviction scores
//     (global memory or LDS);
//   ev_in / ev_out: the pair's eviction bitmap words before / after (may be
//     the same; ev_out == nullptr: the new bitmap is not written);
//   sel_row: the pair's list, sel_cap entries (global memory or LDS);
//   sel_count_slot: where the size goes (nullptr: not written);
//   SWAP with sw.load != nullptr: also form the load / evict lists against
//     the previous selection (global memory).  sw is taken by value: a
//     reference into a kernel's by-value argument would force a stack copy
//     of the whole argument and turn every global access into a flat one.
//   after_loads / after_eviction: called by every thread once the inputs'
//     loads are issued, and once the eviction part is decided (a caller's
//     own memory traffic can go out there without delaying these loads).
struct NoHook {
  __device__ void operator()() const {}
};

// Inlined at every call: a call would pass the hooks' captures, and the
// caller's registers around it, through scratch memory.
template <int R, bool SWAP, class H1 = NoHook, class H2 = NoHook, int NT = kSelThreads>
__device__ __forceinline__ int select_pair(SelSharedT<NT>& sh, int bh, int T, int bs, int max_blocks,
                           const float* __restrict__ sq_row, const float* __restrict__ se_row, int k_e,
                           int k_q, const uint32_t* ev_in, uint32_t* ev_out, int32_t* sel_row, int sel_cap,
                           int32_t* sel_count_slot, const SwapArgs sw, H1 after_loads = H1(),
                           H2 after_eviction = H2()) {
  constexpr int NW = NT / kWave;
  static_assert(R <= 32 && NT % 256 == 0, "selection shape");
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int nb = (T + bs - 1) / bs;
  const float* se = se_row;
  const float* sq = sq_row;
  const bool swap_lists = SWAP && sw.load != nullptr;

  // every load up front, over the whole capacity so they need not wait for
  // seq_lens; blocks >= nb are masked out afterwards.  The loads are
  // unconditional (indices clamped into the table, max_blocks >= 1) so all
  // of them are in flight together: under a branch each group of three
  // would wait for its data before the next group went out.
  uint32_t ke[R], kq[R], ew[R];
  float fe[R], fq[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = min(r * NT + (int)threadIdx.x, max_blocks - 1);
    fe[r] = se[i];
    fq[r] = sq[i];
    ew[r] = ev_in[i >> 5];
  }
  // fused swap lists: the previous selection (capacity sel_cap <= max_blocks,
  // so R entries per thread cover it), loaded with everything else
  int32_t pv[R];
  int n_prev = 0;
  if (swap_lists) {
    const int32_t* pl = sw.prev + (int64_t)bh * sel_cap;
#pragma unroll
    for (int r = 0; r < R; ++r) pv[r] = pl[min(r * NT + (int)threadIdx.x, sel_cap - 1)];
    n_prev = min(max(sw.prev_count[bh], 0), sel_cap);
  }
  after_loads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool in = r * NT + (int)threadIdx.x < max_blocks;
    ke[r] = in ? order_key(fe[r]) : 0u;
    kq[r] = in ? order_key(fq[r]) : 0u;
    ew[r] = in ? ew[r] : 0u;
  }
  uint32_t valid = 0, evm = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = r * NT + threadIdx.x;
    if (i < nb) {
      valid |= 1u << r;
      evm |= ((ew[r] >> (i & 31)) & 1u) << r;
    }
  }
  int phase = 0;

  // --- eviction part: candidates are the never-evicted blocks ------------
  const uint32_t cand_e = valid & ~evm;
  int wave_cand = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) wave_cand += __popcll(__ballot((cand_e >> r) & 1u));
  const int n_cand = block_sum(wave_cand, phase, sh);
  const int n_e = min(k_e, n_cand);
  uint32_t in_e = 0;
  if (n_e == n_cand) in_e = cand_e;
  else if (n_e > 0) radix_top_k<R, NT>(ke, cand_e, n_e, in_e, phase, sh);
  evm |= cand_e & ~in_e;  // every candidate left out is evicted for good
  after_eviction();

  // --- query part: best of the blocks the eviction part did not take ----
  const uint32_t cand_q = valid & ~in_e;
  const int rest = nb - n_e;
  const int n_q = min(k_q, rest);
  uint32_t in_q = 0;
  if (n_q == rest) in_q = cand_q;
  else if (n_q > 0) radix_top_k<R, NT>(kq, cand_q, n_q, in_q, phase, sh);

  // --- outputs: ascending union via ballots, eviction bitmap words ------
  const uint32_t pick = in_e | in_q;
  int32_t* out = sel_row;
  int n_all;  // size of the union
  // the 32-bit words element r of this wave covers: lanes 0 and 32 own them
  auto write_words = [&](int r, uint64_t pmr) {
    const uint64_t em = __ballot((evm >> r) & 1u);
    const uint64_t vm = __ballot((valid >> r) & 1u);
    const int i0 = r * NT + w * kWave + (lane & 32);
    if (ev_out != nullptr && (lane & 31) == 0 && i0 < nb) {  // this lane loaded that word at the start
      const uint32_t e32 = (uint32_t)(em >> (lane & 32));
      const uint32_t v32 = (uint32_t)(vm >> (lane & 32));
      ev_out[i0 >> 5] = (ew[r] & ~v32) | e32;
    }
    if (swap_lists && (lane & 31) == 0 && i0 < max_blocks) sh.pick_bm[i0 >> 5] = (uint32_t)(pmr >> (lane & 32));
  };
  uint64_t pm[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pm[r] = __ballot((pick >> r) & 1u);
    write_words(r, pm[r]);
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) sh.pos[r][w] = __popcll(pm[r]);
  }
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int pos = before + lanes_below(pm[r]);
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const int c = sh.pos[r][ww];
      pos += ww < w ? c : 0;
      before += c;
    }
    if (((pick >> r) & 1u) && pos < sel_cap) out[pos] = r * NT + threadIdx.x;
  }
  n_all = before;

  const int n_sel = min(n_all, sel_cap);
  if (threadIdx.x == 0 && sel_count_slot != nullptr) *sel_count_slot = n_sel;

  if (swap_lists) {
    // load = selected now and not before (index order); evict = before and
    // not now (order of the previous list) -- the set differences of
    // nosa_swap_diff, from the selection still in registers.  pick_bm was
    // filled with the outputs above.
    for (int wd = threadIdx.x; wd < (max_blocks + 31) / 32; wd += NT) sh.prev_bm[wd] = 0u;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int k = r * NT + threadIdx.x;
      if (k < n_prev && pv[r] >= 0 && pv[r] < max_blocks) atomicOr(&sh.prev_bm[pv[r] >> 5], 1u << (pv[r] & 31));
    }
    __syncthreads();
    int32_t* lo = sw.load + (int64_t)bh * sel_cap;
    int32_t* eo = sw.evict + (int64_t)bh * sel_cap;
    // element r: load if picked and not in prev; evict if entry r of prev is
    // live and not picked
    auto masks = [&](int r, uint64_t& lm, uint64_t& em) {
      const int i = r * NT + threadIdx.x;
      const bool in_prev = i < max_blocks && ((sh.prev_bm[min(i, max_blocks - 1) >> 5] >> (i & 31)) & 1u);
      lm = __ballot(((pick >> r) & 1u) && !in_prev);
      const int x = pv[r];
      const bool live = i < n_prev && x >= 0 && x < max_blocks;
      em = __ballot(live && !((sh.pick_bm[live ? x >> 5 : 0] >> (x & 31)) & 1u));
    };
    int bl = 0, be = 0;
    uint64_t lm[R], em[R];
#pragma unroll
    for (int r = 0; r < R; ++r) masks(r, lm[r], em[r]);
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        sh.pos_load[r][w] = __popcll(lm[r]);
        sh.pos_evict[r][w] = __popcll(em[r]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int pl_ = bl + lanes_below(lm[r]), pe = be + lanes_below(em[r]);
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const int cl = sh.pos_load[r][ww], ce = sh.pos_evict[r][ww];
        pl_ += ww < w ? cl : 0;
        pe += ww < w ? ce : 0;
        bl += cl;
        be += ce;
      }
      if (((lm[r] >> lane) & 1u) && pl_ < sel_cap) lo[pl_] = r * NT + threadIdx.x;
      if (((em[r] >> lane) & 1u) && pe < sel_cap) eo[pe] = pv[r];
    }
    if (threadIdx.x == 0) {
      sw.load_count[bh] = min(bl, sel_cap);
      sw.evict_count[bh] = min(be, sel_cap);
    }
  }
  return n_sel;
}

// ---------------------------------------------------------------------------
// The query part of the selection, and the outputs, made by ONE wave for the
// step where the eviction part has nothing to choose: the never-evicted
// blocks below nb number n_e <= k_e, so every one of them stays in the
// eviction part and none is evicted (the incoming bitmap is the outgoing
// one).  The query part is then the k_q best of the other blocks by
// (score_q desc, index asc), and the results equal select_pair's bit for
// bit.  No workgroup barrier: the decode's other waves stream the eviction
// part's pages meanwhile.
//
// Element r of lane l is block i = r * 64 + l (R * 64 >= max_blocks); rows
// r >= ceil(nb / 64) hold no block and are skipped.  The inputs are loaded
// first (load_query_wave), as early as the caller can issue them.
// ---------------------------------------------------------------------------
// Bit r of a row mask is row r of a lane (R <= 64 rows).
template <int R>
using RowMask = typename std::conditional<(R > 32), uint64_t, uint32_t>::type;

template <int R>
struct QueryWaveInputs {
  float fq[R];      // score_q of the wave's elements (clamped indices)
  int32_t pv[R];    // entries of the previous selection
  int n_prev;
};

// sq_row: the pair's max_blocks query-aware scores (global memory or LDS).
template <int R>
__device__ __forceinline__ void load_query_wave(QueryWaveInputs<R>& in, int bh, int max_blocks,
                                                const float* __restrict__ sq_row, int sel_cap, const SwapArgs& sw) {
  const int lane = threadIdx.x % kWave;
  const float* sq = sq_row;
#pragma unroll
  for (int r = 0; r < R; ++r) in.fq[r] = sq[min(r * kWave + lane, max_blocks - 1)];
  in.n_prev = 0;
  if (sw.load != nullptr) {
    const int32_t* pl = sw.prev + (int64_t)bh * sel_cap;
#pragma unroll
    for (int r = 0; r < R; ++r) in.pv[r] = pl[min(r * kWave + lane, sel_cap - 1)];
    in.n_prev = min(max(sw.prev_count[bh], 0), sel_cap);
  }
}

// Marks in `out` (bit r) the k best of the elements in `cand` under (key
// desc, index asc), by one wave: a radix select over 8-bit digits from the
// highest bit in which the candidates' keys differ, counting digits in an
// LDS histogram (hist: 256 words of this wave) and finding the bin of the
// k-th key with a wave prefix sum; exact ties at the end go to the lowest
// indices.  Requires 0 < k < number of candidates; rows >= nr hold none.
template <int R>
__device__ __forceinline__ void wave_radix_top_k(const uint32_t (&key)[R], RowMask<R> cand, int k, int nr,
                                                 uint32_t* hist, RowMask<R>& out) {
  const int lane = threadIdx.x % kWave;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (r < nr && ((cand >> r) & 1u)) {
      kmin = min(kmin, key[r]);
      kmax = max(kmax, key[r]);
    }
  kmin = xor_reduce<1, kWave>(kmin, [](uint32_t x, uint32_t y) { return min(x, y); });
  kmax = xor_reduce<1, kWave>(kmax, [](uint32_t x, uint32_t y) { return max(x, y); });
  int hi = kmin == kmax ? 0 : 32 - __clz(kmin ^ kmax);  // bits [hi, 32) are shared
  uint32_t prefix = hi >= 32 ? 0u : kmin & ~((1u << hi) - 1u);
  uint32_t pmask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
  int rem = k, n_eq = 0;
  bool done = false;
  while (hi > 0 && !done) {
    const int lo = hi > 8 ? hi - 8 : 0;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[lane + kWave * j] = 0u;
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < nr && ((cand >> r) & 1u) && (key[r] & pmask) == prefix) atomicAdd(&hist[(key[r] >> lo) & dmask], 1u);
    wave_lds_sync();
    // lane l holds digits 255 - 4l .. 252 - 4l (descending); keys with a
    // digit above this lane's are counted before it
    uint32_t c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = hist[255 - 4 * lane - e];
    const int c4 = (int)(c[0] + c[1] + c[2] + c[3]);
    int cum = wave_scan_incl(c4) - c4;
    int dg = -1, above = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (dg < 0 && c[e] > 0 && cum + (int)c[e] >= rem) {
        dg = 255 - 4 * lane - e;
        above = cum;
        eq = (int)c[e];
      }
      cum += (int)c[e];
    }
    const uint64_t hit = __ballot(dg >= 0);
    const int src = __ffsll((unsigned long long)hit) - 1;
    const uint32_t digit = (uint32_t)__builtin_amdgcn_readlane(dg, src);
    rem -= __builtin_amdgcn_readlane(above, src);
    n_eq = __builtin_amdgcn_readlane(eq, src);
    wave_lds_sync();  // the histogram is cleared again by the next pass
    prefix |= digit << lo;
    pmask |= dmask << lo;
    hi = lo;
    done = rem == n_eq;  // the whole bin is taken: prefix is the threshold
  }
  if (rem == n_eq) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < nr && ((cand >> r) & 1u) && (key[r] & pmask) >= prefix) out |= RowMask<R>(1) << r;
    return;
  }
  // exact key ties at the threshold: the rem lowest block indices win
  int before = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < nr) {
      const bool c_ = (cand >> r) & 1u;
      const uint64_t eqm = __ballot(c_ && key[r] == prefix);
      const int rank = before + lanes_below(eqm);
      before += __popcll(eqm);
      if (c_ && (key[r] > prefix || (key[r] == prefix && rank < rem))) out |= RowMask<R>(1) << r;
    }
  }
}

//   evw, evw2: this lane's words lane and lane + 64 of the incoming bitmap
//     (words past ceil(max_blocks/32) all ones; evw2 is read for R > 32);
//   ev_out: the pairs' outgoing bitmaps (the pair's words < nb are written);
//   sel_row / sel_count_slot: the ascending union and its size (nullptr:
//     not written);
//   sw: swap lists against the previous selection (sw.load == nullptr: none);
//   hist, pick_bm, prev_bm: LDS scratch of this wave (256 and
//     ceil(max_blocks/32) words);
//   qlist: receives the query part's blocks, ascending (LDS).
// Returns the union's size (capped at sel_cap), the same in every lane.
template <int R>
__device__ __forceinline__ int select_query_wave(const QueryWaveInputs<R>& in, int bh, int nb, int max_blocks, int k_q,
                                 uint32_t evw, uint32_t evw2, int n_e, uint32_t* ev_out, int32_t* sel_row, int sel_cap,
                                 int32_t* sel_count_slot, const SwapArgs& sw, uint32_t* hist, uint32_t* pick_bm,
                                 uint32_t* prev_bm, int32_t* qlist) {
  static_assert(R <= 64, "rows of a lane: at most two bitmap words per lane");
  const int lane = threadIdx.x % kWave;
  const bool swap_lists = sw.load != nullptr;
  const int nr = min((nb + kWave - 1) / kWave, R);  // rows holding blocks
  // eviction part = the never-evicted blocks; the query part's candidates
  RowMask<R> in_e = 0, cand = 0;
  uint32_t key[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = r * kWave + lane;
    const uint32_t src = r < 32 ? evw : evw2;  // rows 32.. hold words 64..
    const uint32_t wlo = (uint32_t)__builtin_amdgcn_readlane((int)src, (2 * r) & 63);
    const uint32_t whi = (uint32_t)__builtin_amdgcn_readlane((int)src, (2 * r + 1) & 63);
    const uint32_t word = lane < 32 ? wlo : whi;
    const bool valid = i < nb;
    const bool e = valid && !((word >> (lane & 31)) & 1u);
    in_e |= RowMask<R>(e) << r;
    cand |= RowMask<R>(valid && !e) << r;
    key[r] = order_key(in.fq[r]);
  }
  const int n_avail = nb - n_e;
  const int kk = min(k_q, n_avail);
  RowMask<R> in_q = 0;
  if (kk >= n_avail) in_q = cand;
  else if (kk > 0) wave_radix_top_k<R>(key, cand, kk, nr, hist, in_q);

  // outputs: the ascending union, the query part's list, the bitmap words
  const RowMask<R> pick = in_e | in_q;
  uint64_t pm[R];
  int n_all = 0, n_q = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pm[r] = 0;
    if (r < nr) {
      const int i = r * kWave + lane;
      pm[r] = __ballot((pick >> r) & 1u);
      const int pos = n_all + lanes_below(pm[r]);
      if (sel_row != nullptr && ((pick >> r) & 1u) && pos < sel_cap) sel_row[pos] = i;
      n_all += __popcll(pm[r]);
      const uint64_t qm = __ballot((in_q >> r) & 1u);
      if ((in_q >> r) & 1u) qlist[n_q + lanes_below(qm)] = i;
      n_q += __popcll(qm);
    }
  }
  const int n_sel = min(n_all, sel_cap);
  if (lane == 0 && sel_count_slot != nullptr) *sel_count_slot = n_sel;
  const int words = (max_blocks + 31) / 32;
  if (ev_out != nullptr && lane < words && lane * 32 < nb) ev_out[(int64_t)bh * words + lane] = evw;
  if (R > 32 && ev_out != nullptr && lane + kWave < words && (lane + kWave) * 32 < nb)
    ev_out[(int64_t)bh * words + kWave + lane] = evw2;

  if (swap_lists) {
    // membership bitmaps of the union and of the previous selection
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (lane == 0 && 2 * r < words) {
        pick_bm[2 * r] = (uint32_t)pm[r];
        if (2 * r + 1 < words) pick_bm[2 * r + 1] = (uint32_t)(pm[r] >> 32);
      }
    for (int wd = lane; wd < words; wd += kWave) prev_bm[wd] = 0u;
    wave_lds_sync();
    const int nrp = (in.n_prev + kWave - 1) / kWave;  // rows holding previous entries
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int k = r * kWave + lane;
      if (r < nrp && k < in.n_prev && in.pv[r] >= 0 && in.pv[r] < max_blocks)
        atomicOr(&prev_bm[in.pv[r] >> 5], 1u << (in.pv[r] & 31));
    }
    wave_lds_sync();
    // load = picked and not before (index order); evict = before and not
    // picked (the previous list's order)
    int32_t* lo = sw.load + (int64_t)bh * sel_cap;
    int32_t* eo = sw.evict + (int64_t)bh * sel_cap;
    int bl = 0, be = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < nr) {
        const int i = r * kWave + lane;
        const bool in_prev = (prev_bm[min(i, max_blocks - 1) >> 5] >> (i & 31)) & 1u;
        const uint64_t lm = __ballot(((pick >> r) & 1u) && !in_prev);
        const int pl_ = bl + lanes_below(lm);
        if (((lm >> lane) & 1u) && pl_ < sel_cap) lo[pl_] = i;
        bl += __popcll(lm);
      }
      if (r < nrp) {
        const int k = r * kWave + lane;
        const int x = in.pv[r];
        const bool live = k < in.n_prev && x >= 0 && x < max_blocks;
        const uint64_t em = __ballot(live && !((pick_bm[live ? x >> 5 : 0] >> (x & 31)) & 1u));
        const int pe = be + lanes_below(em);
        if (((em >> lane) & 1u) && pe < sel_cap) eo[pe] = x;
        be += __popcll(em);
      }
    }
    if (lane == 0) {
      sw.load_count[bh] = min(bl, sel_cap);
      sw.evict_count[bh] = min(be, sel_cap);
    }
  }
  return n_sel;
}

}  // namespace nosa
