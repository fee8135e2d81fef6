// Selection kernels: dual selection per (b, h) (select_pair, with or
// without the fused swap lists) and the standalone block-swap set
// differences [NOSA summary (gist.science 2510.13602), Methodology 2
// (NOSI): set differences between consecutive block sets drive block
// swapping].

#include "nosa_launch.hpp"
#include "nosa_select_impl.hpp"

namespace nosa {

// One workgroup of NT threads per (b, h).
template <int R, bool SWAP, int NT>
__global__ __launch_bounds__(NT) void select_kernel(int Hkv, int bs, int max_blocks,
                                                            const float* __restrict__ score_q,
                                                            const float* __restrict__ score_e,
                                                            const int32_t* __restrict__ seq_lens, int k_e, int k_q,
                                                            uint32_t* __restrict__ evicted,
                                                            int32_t* __restrict__ sel, int sel_cap,
                                                            int32_t* __restrict__ sel_count, const SwapArgs sw) {
  __shared__ SelSharedT<NT> sh;
  const int bh = blockIdx.x;
  const int T = min(max(seq_lens[bh / Hkv], 0), max_blocks * bs);
  uint32_t* ev = evicted + (int64_t)bh * ((max_blocks + 31) / 32);
  select_pair<R, SWAP, NoHook, NoHook, NT>(sh, bh, T, bs, max_blocks, score_q + (int64_t)bh * max_blocks,
                                           score_e + (int64_t)bh * max_blocks, k_e, k_q, ev, ev,
                                           sel + (int64_t)bh * sel_cap, sel_cap, sel_count + bh, sw);
}

// One wave per (b, h); membership through an LDS bitmap, order-preserving
// compaction through ballots.  The first 64 entries of both lists are
// loaded with the counts (clamped, branch-free), so short lists cost one
// memory round trip.
__global__ __launch_bounds__(kWave) void swap_diff_kernel(int max_blocks, int cap,
                                                          const int32_t* __restrict__ prev,
                                                          const int32_t* __restrict__ prev_count,
                                                          const int32_t* __restrict__ cur,
                                                          const int32_t* __restrict__ cur_count,
                                                          int32_t* __restrict__ load,
                                                          int32_t* __restrict__ load_count,
                                                          int32_t* __restrict__ evict,
                                                          int32_t* __restrict__ evict_count) {
  __shared__ uint32_t bm[2][kMaxBlocks / 32];  // [0]: prev, [1]: cur
  const int bh = blockIdx.x;
  const int lane = threadIdx.x;
  const int32_t* lst[2] = {prev + (int64_t)bh * cap, cur + (int64_t)bh * cap};
  const int first = min(lane, cap - 1);
  const int x0[2] = {lst[0][first], lst[1][first]};
  const int n[2] = {min(max(prev_count[bh], 0), cap), min(max(cur_count[bh], 0), cap)};
  for (int w = lane; w < kMaxBlocks / 32; w += kWave) bm[0][w] = bm[1][w] = 0u;
  wave_lds_sync();
  // mark both lists
#pragma unroll
  for (int li = 0; li < 2; ++li) {
    for (int base = 0; base < n[li]; base += kWave) {
      const int k = base + lane;
      const int x = base == 0 ? x0[li] : (k < n[li] ? lst[li][k] : -1);
      if (k < n[li] && x >= 0 && x < max_blocks) atomicOr(&bm[li][x >> 5], 1u << (x & 31));
    }
  }
  wave_lds_sync();
  // load = cur \ prev (li = 1 tested against 0), evict = prev \ cur
#pragma unroll
  for (int li = 0; li < 2; ++li) {
    const int tl = 1 - li;  // list under test: cur first, then prev
    int32_t* out = (li == 0 ? load : evict) + (int64_t)bh * cap;
    int n_out = 0;
    for (int base = 0; base < n[tl]; base += kWave) {
      const int k = base + lane;
      const int x = base == 0 ? x0[tl] : (k < n[tl] ? lst[tl][k] : -1);
      const bool keep = k < n[tl] && x >= 0 && x < max_blocks && !((bm[li][x >> 5] >> (x & 31)) & 1u);
      const uint64_t mk = __ballot(keep);
      if (keep) out[n_out + lanes_below(mk)] = x;
      n_out += __popcll(mk);
    }
    if (lane == 0) (li == 0 ? load_count : evict_count)[bh] = n_out;
  }
}

static hipError_t launch_select_any(const nosa_dims& d, const float* score_q, const float* score_e,
                                    const int32_t* seq_lens, int32_t k_e, int32_t k_q, uint32_t* evicted,
                                    int32_t* sel, int32_t sel_cap, int32_t* sel_count, const SwapArgs* sw,
                                    hipStream_t stream) {
  const dim3 grid(d.batch * d.n_kv_heads);
  const SwapArgs none = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  const SwapArgs args = sw ? *sw : none;
#define NOSA_SELECT(RR, NT)                                                                                    \
  do {                                                                                                         \
    if (sw)                                                                                                    \
      select_kernel<RR, true, NT><<<grid, NT, 0, stream>>>(d.n_kv_heads, d.block_size, d.max_blocks, score_q,  \
                                                           score_e, seq_lens, k_e, k_q, evicted, sel, sel_cap, \
                                                           sel_count, args);                                   \
    else                                                                                                       \
      select_kernel<RR, false, NT><<<grid, NT, 0, stream>>>(d.n_kv_heads, d.block_size, d.max_blocks,          \
                                                            score_q, score_e, seq_lens, k_e, k_q, evicted, sel, \
                                                            sel_cap, sel_count, args);                         \
  } while (0)
  // Up to 2,048 blocks: four waves, R keys per thread.  Beyond, sixteen
  // waves: the selection's time follows the keys each thread walks (every
  // pass of the radix select loops over them), so a wider workgroup with
  // fewer keys per thread is faster there despite its costlier barriers.
  const int R = (d.max_blocks + kSelThreads - 1) / kSelThreads;  // keys per thread of four waves
  const int RW = (d.max_blocks + 1023) / 1024;                   // keys per thread of sixteen waves
  if (R <= 2) NOSA_SELECT(2, 256);
  else if (R <= 4) NOSA_SELECT(4, 256);
  else if (R <= 8) NOSA_SELECT(8, 256);
  else if (RW <= 3) NOSA_SELECT(3, 1024);
  else if (RW <= 4) NOSA_SELECT(4, 1024);
  else NOSA_SELECT(8, 1024);
#undef NOSA_SELECT
  return hipGetLastError();
}

hipError_t launch_select(const nosa_dims& d, const float* score_q, const float* score_e,
                         const int32_t* seq_lens, int32_t k_e, int32_t k_q, uint32_t* evicted,
                         int32_t* sel, int32_t sel_cap, int32_t* sel_count, hipStream_t stream) {
  return launch_select_any(d, score_q, score_e, seq_lens, k_e, k_q, evicted, sel, sel_cap, sel_count, nullptr,
                           stream);
}

hipError_t launch_select_swap(const nosa_dims& d, const float* score_q, const float* score_e,
                              const int32_t* seq_lens, int32_t k_e, int32_t k_q, uint32_t* evicted,
                              int32_t* sel, int32_t sel_cap, int32_t* sel_count, const int32_t* prev,
                              const int32_t* prev_count, int32_t* load, int32_t* load_count, int32_t* evict,
                              int32_t* evict_count, hipStream_t stream) {
  const SwapArgs sw = {prev, prev_count, load, load_count, evict, evict_count};
  return launch_select_any(d, score_q, score_e, seq_lens, k_e, k_q, evicted, sel, sel_cap, sel_count, &sw,
                           stream);
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
