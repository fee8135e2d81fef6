// Index side of the step: writing tokens into pages and keeping the
// sub-block summaries that block scoring pools over.
//
// Sources: NOSA summary (gist.science 2510.13602), Methodology 1, bullet
// on the block-wise implementation (two-stage pooling: mean inside a
// sub-block, max over a block) and Methodology 2 (NOSI fuses pooling into
// the index-side kernel; the KV cache is kept in block-sized units); Spin
// summary (gist.science 2604.26837), 2.A (Index as its own operation) and
// 2.B (per-head physical pages).
//
// A summary entry is the mean of its sub-block's present tokens: bf16 keys
// and fp32 logits are summed in float64 in ascending token order (exact for
// bf16 keys) and rounded once to fp32, so nosa_build_summaries and
// nosa_append produce bit-identical entries for the same tokens.

#include "nosa_launch.hpp"
#include "nosa_summary.hpp"

namespace nosa {

Table make_table(const nosa_dims& d, const nosa_kv& kv) {
  Table t;
  t.kind = kv.kind;
  t.Hkv = d.n_kv_heads;
  t.max_blocks = d.max_blocks;
  t.dir_entries = kv.dir_entries;
  t.seg_log2 = kv.seg_log2;
  t.blocks_log2 = kv.blocks_log2;
  t.num_pages = kv.num_pages;
  t.num_segments = kv.num_segments;
  t.table = kv.table;
  t.directory = kv.directory;
  t.segments = kv.segments;
  t.packed = kv.packed;
  t.err = kv.err_flags;
  return t;
}

// ---------------------------------------------------------------------------
// prefill: contiguous [B][Hkv][src_tokens][D] sources -> pages.
// One workgroup per (logical block, (b, h)).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void prefill_kernel(Table t, int bs, const uint16_t* __restrict__ k_src,
                                                      const uint16_t* __restrict__ v_src,
                                                      const float* __restrict__ e_src, int src_tokens,
                                                      const int32_t* __restrict__ seq_lens,
                                                      uint16_t* __restrict__ k_pages,
                                                      uint16_t* __restrict__ v_pages,
                                                      float* __restrict__ e_pages) {
  const int i = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / t.Hkv;
  const int T = seq_lens[b];
  if (T < 0 || T > src_tokens || T > t.max_blocks * bs) {
    if (i == 0 && threadIdx.x == 0) flag_error(t.err);
    return;
  }
  const int t0 = i * bs;
  if (t0 >= T) return;
  const int ntok = min(bs, T - t0);
  uint32_t doc;
  const int64_t page = page_of_any(t, bh, i, doc);
  if (page < 0) {
    if (threadIdx.x == 0) flag_error(t.err);
    return;
  }
  const uint16_t* ks = k_src + ((int64_t)bh * src_tokens + t0) * D;
  const uint16_t* vs = v_src + ((int64_t)bh * src_tokens + t0) * D;
  const float* es = e_src + (int64_t)bh * src_tokens + t0;
  uint4* kp = reinterpret_cast<uint4*>(k_pages + page * (int64_t)bs * D);
  uint4* vp = reinterpret_cast<uint4*>(v_pages + page * (int64_t)bs * D);

  // K page [D/8][bs][8]: item (octet o, token tok) is one 16-byte row piece.
  for (int it = threadIdx.x; it < (D / 8) * bs; it += blockDim.x) {
    const int o = it / bs, tok = it % bs;
    if (tok < ntok) kp[o * bs + tok] = *reinterpret_cast<const uint4*>(ks + (int64_t)tok * D + o * 8);
  }
  // V page [bs/8][D][8]: item (token octet to, dim d) gathers 8 tokens.
  for (int it = threadIdx.x; it < (bs / 8) * D; it += blockDim.x) {
    const int to = it / D, d = it % D;
    if (to * 8 >= ntok) continue;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ta = to * 8 + 2 * j, tb = ta + 1;
      const uint32_t lo = ta < ntok ? vs[(int64_t)ta * D + d] : 0u;
      const uint32_t hi = tb < ntok ? vs[(int64_t)tb * D + d] : 0u;
      w[j] = lo | (hi << 16);
    }
    vp[to * D + d] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  for (int tok = threadIdx.x; tok < ntok; tok += blockDim.x) e_pages[page * bs + tok] = es[tok];
}

// build_summaries: one thread per (sub-block, d-quad); threads with u == 0
// also take the logit mean.
template <int D>
__global__ __launch_bounds__(256) void summaries_kernel(Table t, int bs, int ss,
                                                        const int32_t* __restrict__ seq_lens,
                                                        const uint16_t* __restrict__ k_pages,
                                                        const float* __restrict__ e_pages,
                                                        float* __restrict__ k_summary,
                                                        float* __restrict__ e_summary) {
  constexpr int NQ = D / 4;
  constexpr int SPB = 256 / NQ;  // sub-blocks per workgroup
  const int bh = blockIdx.y;
  const int b = bh / t.Hkv;
  const int nsub = bs / ss;
  const int CS = t.max_blocks * nsub;
  const int T = min(max(seq_lens[b], 0), t.max_blocks * bs);
  const int s = blockIdx.x * SPB + threadIdx.x / NQ;
  const int u = threadIdx.x % NQ;
  if (s >= CS) return;
  const int i = s / nsub, j = s % nsub;
  const int lo = i * bs + j * ss;
  if (lo >= T) return;
  const int hi = min(lo + ss, T);
  uint32_t doc;
  const int64_t page = page_of_any(t, bh, i, doc);
  if (page < 0) {
    if (u == 0) flag_error(t.err);
    return;
  }
  const double inv_n = 1.0 / (double)(hi - lo);
  double a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  sum_key_quad<D>(k_pages + page * (int64_t)bs * D, bs, u, lo - i * bs, hi - i * bs, a0, a1, a2, a3);
  float4 r;
  r.x = (float)(a0 * inv_n);
  r.y = (float)(a1 * inv_n);
  r.z = (float)(a2 * inv_n);
  r.w = (float)(a3 * inv_n);
  reinterpret_cast<float4*>(k_summary)[((int64_t)bh * NQ + u) * CS + s] = r;
  if (u == 0) {
    const double ae = sum_logits(e_pages + page * bs, lo - i * bs, hi - i * bs);
    e_summary[(int64_t)bh * CS + s] = (float)(ae * inv_n);
  }
}

// ---------------------------------------------------------------------------
// append: one workgroup per sequence, one wave per KV head.  Wave h writes
// token T of (b, h) into its page and recomputes the summary of the
// sub-block holding it (older tokens from the page, the new one from the
// input, ascending order); the workgroup then advances seq_lens[b].  The new
// token's loads go out before the position is known, so the kernel costs
// three dependent memory round trips: position, page, older tokens.
// ---------------------------------------------------------------------------
template <int D>
__global__ void append_kernel(Table t, int bs, int ss, const uint16_t* __restrict__ k_new,
                              const uint16_t* __restrict__ v_new, const float* __restrict__ e_new,
                              int32_t* __restrict__ seq_lens, uint16_t* __restrict__ k_pages,
                              uint16_t* __restrict__ v_pages, float* __restrict__ e_pages,
                              float* __restrict__ k_summary, float* __restrict__ e_summary) {
  constexpr int NQ = D / 4;
  constexpr int VL = D / kWave;  // value dims per lane
  const int b = blockIdx.x;
  const int h = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int bh = b * t.Hkv + h;
  const int nsub = bs / ss;
  const int CS = t.max_blocks * nsub;
  const uint16_t* kn = k_new + (int64_t)bh * D;
  const uint16_t* vn = v_new + (int64_t)bh * D;
  const uint4 k_oct = reinterpret_cast<const uint4*>(kn)[lane % (D / 8)];
  const uint2 k_quad = reinterpret_cast<const uint2*>(kn)[lane % NQ];
  uint16_t v_dim[VL];
#pragma unroll
  for (int j = 0; j < VL; ++j) v_dim[j] = vn[lane + j * kWave];
  const float e_tok = e_new[bh];
  const int pos = seq_lens[b];
  const bool in_range = pos >= 0 && pos < t.max_blocks * bs;
  if (in_range) {
    const int i = pos / bs, r = pos % bs;
    uint32_t doc;
    const int64_t page = page_of_any(t, bh, i, doc);
    if (page < 0) {
      if (lane == 0) flag_error(t.err);
    } else {
      uint16_t* kpage = k_pages + page * (int64_t)bs * D;
      uint16_t* vpage = v_pages + page * (int64_t)bs * D;
      const int j = r / ss;
      const int lo = j * ss;  // page-relative start of the sub-block
      const double inv_n = 1.0 / (double)(r - lo + 1);
      const int s = i * nsub + j;
      if (lane < NQ) {
        double a0 = 0, a1 = 0, a2 = 0, a3 = 0;
        sum_key_quad<D>(kpage, bs, lane, lo, r, a0, a1, a2, a3);
        a0 += (double)bf16_lo(k_quad.x);
        a1 += (double)bf16_hi(k_quad.x);
        a2 += (double)bf16_lo(k_quad.y);
        a3 += (double)bf16_hi(k_quad.y);
        float4 o;
        o.x = (float)(a0 * inv_n);
        o.y = (float)(a1 * inv_n);
        o.z = (float)(a2 * inv_n);
        o.w = (float)(a3 * inv_n);
        reinterpret_cast<float4*>(k_summary)[((int64_t)bh * NQ + lane) * CS + s] = o;
      }
      if (lane == NQ) {  // the logit mean runs beside the key quads
        double ae = sum_logits(e_pages + page * bs, lo, r);
        ae += (double)e_tok;
        e_summary[(int64_t)bh * CS + s] = (float)(ae * inv_n);
      }
      // the new token itself (after the reads of the older ones above)
      if (lane < D / 8) reinterpret_cast<uint4*>(kpage)[lane * bs + r] = k_oct;
#pragma unroll
      for (int jj = 0; jj < VL; ++jj) vpage[((r / 8) * D + lane + jj * kWave) * 8 + r % 8] = v_dim[jj];
      if (lane == 0) e_pages[page * bs + r] = e_tok;
    }
  } else if (threadIdx.x == 0) {
    flag_error(t.err);
  }
  __syncthreads();
  if (threadIdx.x == 0 && in_range) seq_lens[b] = pos + 1;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_prefill(const nosa_dims& d, const nosa_kv& kv, const uint16_t* k_src,
                          const uint16_t* v_src, const float* e_src, int32_t src_tokens,
                          const int32_t* seq_lens, hipStream_t stream) {
  const Table t = make_table(d, kv);
  const dim3 grid(d.max_blocks, d.batch * d.n_kv_heads);
  if (d.head_dim == 128)
    prefill_kernel<128><<<grid, 256, 0, stream>>>(t, d.block_size, k_src, v_src, e_src, src_tokens,
                                                  seq_lens, kv.k_pages, kv.v_pages, kv.e_pages);
  else
    prefill_kernel<64><<<grid, 256, 0, stream>>>(t, d.block_size, k_src, v_src, e_src, src_tokens,
                                                 seq_lens, kv.k_pages, kv.v_pages, kv.e_pages);
  return hipGetLastError();
}

hipError_t launch_build_summaries(const nosa_dims& d, const nosa_kv& kv, const int32_t* seq_lens,
                                  float* k_summary, float* e_summary, hipStream_t stream) {
  const Table t = make_table(d, kv);
  const int CS = d.max_blocks * (d.block_size / d.sub_block);
  const int spb = 256 / (d.head_dim / 4);
  const dim3 grid((CS + spb - 1) / spb, d.batch * d.n_kv_heads);
  if (d.head_dim == 128)
    summaries_kernel<128><<<grid, 256, 0, stream>>>(t, d.block_size, d.sub_block, seq_lens, kv.k_pages,
                                                    kv.e_pages, k_summary, e_summary);
  else
    summaries_kernel<64><<<grid, 256, 0, stream>>>(t, d.block_size, d.sub_block, seq_lens, kv.k_pages,
                                                   kv.e_pages, k_summary, e_summary);
  return hipGetLastError();
}

hipError_t launch_append(const nosa_dims& d, const nosa_kv& kv, const uint16_t* k_new,
                         const uint16_t* v_new, const float* e_new, int32_t* seq_lens,
                         float* k_summary, float* e_summary, hipStream_t stream) {
  const Table t = make_table(d, kv);
  const dim3 grid(d.batch), block(kWave * d.n_kv_heads);
  if (d.head_dim == 128)
    append_kernel<128><<<grid, block, 0, stream>>>(t, d.block_size, d.sub_block, k_new, v_new, e_new,
                                                   seq_lens, kv.k_pages, kv.v_pages, kv.e_pages,
                                                   k_summary, e_summary);
  else
    append_kernel<64><<<grid, block, 0, stream>>>(t, d.block_size, d.sub_block, k_new, v_new, e_new,
                                                  seq_lens, kv.k_pages, kv.v_pages, kv.e_pages,
                                                  k_summary, e_summary);
  return hipGetLastError();
}

}  // namespace nosa
