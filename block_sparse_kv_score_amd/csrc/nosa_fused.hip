// Append and block scoring in one launch (nosa_append_score).
//
// The two stages are those of nosa_append and nosa_score_blocks, with the
// same arithmetic, so the results are bit-identical to the two separate
// calls:
//   * append [NOSA summary (gist.science 2510.13602), Methodology 2: NOSI
//     fuses pooling into the index-side kernel]: the new token goes into its
//     page and the summary of its sub-block is recomputed (float64 sums in
//     ascending token order, one rounding to fp32);
//   * scoring [Methodology 1, block-wise implementation]: sub-block mean
//     summaries dotted with the group's mean query, max over each block,
//     and the eviction logits pooled the same way.
//
// Layout of the launch.  Grid (chunks of SPG sub-blocks, B * Hkv), 256
// threads, as the score kernel, with the chunks of a pair taken last to
// first: the chunk holding the new token is the last non-empty one, so its
// "lead" workgroup is the first of the pair to be dispatched and the
// append's dependent loads (position, page, older tokens) overlap the
// streaming of the pair's other chunks.  (Starting every pair's append at
// once, at the head of the launch, measured slower: the appends then
// compete with each other.)  The lead workgroup scores its own chunk with
// the new summary from LDS; no other workgroup reads what the append
// writes.
//
// The new length is written to a second buffer (seq_lens_out), never to
// the one every workgroup reads (seq_lens_in), so no reader can see it
// early.
//
// Deferred RoPE (packed table; scoring only).  Stored keys carry only their
// in-document rotation (LazyAttention summary, 2. Decoding), so the
// query-aware score of a block in the document starting at position st is
// taken with the group's mean query turned by (n - st): by linearity of the
// rotation and the mean, Rot(n - st) qbar . kbar_stored equals the mean of
// Rot(n) q_g . Rot(st) k over the sub-block.  The workgroup turns the mean
// query once per distinct document among its blocks (float64, one sincos
// per lane; documents span many blocks, so usually once) and keeps the
// results in LDS.
//
// QKV input (nosa_append_score_qkv; NOSA summary, Methodology 2: NOSI fuses
// the eviction head, the QKV split and pooling into one kernel).  The new
// token arrives as each sequence's fused projection row [q | k | v]; k and v
// are read from the row, the eviction logit is the head's w_h . v (float64,
// one rounding to fp32), the group's query for scoring comes from the row,
// and one workgroup per pair writes the split query out for the decode.

#include "nosa_launch.hpp"
#include "nosa_summary.hpp"

namespace nosa {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kFusedThreads = 256;
constexpr int kStageTok = 32;  // older tokens staged through LDS per pass
constexpr int kRopeBlocksPerWave = 4;  // RoPE scoring: nsub >= 4 (SPW / nsub blocks per wave)

struct FusedArgs {
  Table t;
  int Hq, bs, ss;
  // append (k_new == nullptr: no append)
  const uint16_t* k_new;
  const uint16_t* v_new;
  const float* e_new;
  uint16_t* k_pages;
  uint16_t* v_pages;
  float* e_pages;
  const int32_t* seq_in;
  int32_t* seq_out;
  float* k_summary;
  float* e_summary;
  // scoring
  const uint16_t* q;
  float* score_q;
  float* score_e;
  // deferred RoPE (packed table): query positions [B] and the base
  const int32_t* q_pos;
  double rope_base;
  // QKV input (QKV variants): fused projection rows, eviction head, split query
  const uint16_t* qkv;   // [B][(Hq + 2 Hkv) D]
  const float* w_evict;  // [Hkv][D]
  uint16_t* q_out;       // [B][Hq][D]
};

// The group's mean query turned by (n - start) for each distinct document
// among the workgroup's blocks (RoPE scoring): rq[r] for document r, didx
// the document of each block, dst each document's start (blocks).
template <int D, bool ROPE>
struct RopeSmem {
  double rq[kFusedThreads / kWave * kRopeBlocksPerWave][D];
  uint32_t docb[kFusedThreads / kWave * kRopeBlocksPerWave];
  int didx[kFusedThreads / kWave * kRopeBlocksPerWave];
  uint32_t dst[kFusedThreads / kWave * kRopeBlocksPerWave];
  int ndoc;
};
template <int D>
struct RopeSmem<D, false> {};

// NST: older tokens staged per pass (1 where the kernel never appends)
template <int D, int NST>
struct FusedSmem {
  double qbar[D];
  f4 knew[D / 4];  // the new token's sub-block summary (append workgroup)
  uint4 kold[NST][D / 8];  // staged older keys of that sub-block
  float eold[NST];
  float enew;
  int have_new;
};

// The append of pair bh, by the whole append workgroup (uniform call):
// token position pos (in range), page the page of its block (-1: none).  The older tokens of the new token's
// sub-block are staged through LDS NST at a time by all threads (one
// memory round trip per pass instead of one per batch of a single lane);
// wave 0 then sums them in ascending token order exactly as sum_key_quad /
// sum_logits do, adds the new token, and writes the summary (global memory
// and sh.knew / sh.enew) and the token itself.  Mirrors append_kernel.
template <int D, int NST>
__device__ void append_token(const FusedArgs& a, FusedSmem<D, NST>& sh, int bh, int pos, int64_t page,
                             const uint16_t* kn, const uint16_t* vn, float e_new) {
  constexpr int NQ = D / 4;
  constexpr int NO = D / 8;  // 16-byte octets per key row
  constexpr int VL = D / kWave;
  constexpr int IPT = (NO * NST + kFusedThreads - 1) / kFusedThreads;  // staged items per thread
  const Table& t = a.t;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int bs = a.bs, ss = a.ss, nsub = bs / ss, CS = t.max_blocks * nsub;
  const int i = pos / bs, r = pos % bs;
  const int j = r / ss;
  const int lo = j * ss;  // page-relative start of the sub-block
  if (page < 0) {
    if (threadIdx.x == 0) flag_error(t.err);
    return;
  }
  uint16_t* kpage = a.k_pages + page * (int64_t)bs * D;
  uint16_t* vpage = a.v_pages + page * (int64_t)bs * D;
  float* epage = a.e_pages + page * bs;
  double a0 = 0, a1 = 0, a2 = 0, a3 = 0, ae = 0;
  for (int t0 = lo; t0 < r; t0 += NST) {  // uniform trip count
    const int n = min(NST, r - t0);
    uint4 kv[IPT];
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int it = min((int)threadIdx.x + u * kFusedThreads, NO * n - 1);  // clamped: no branch
      const int o = it / n, tt = it % n;
      kv[u] = reinterpret_cast<const uint4*>(kpage)[o * bs + t0 + tt];
    }
    const float ev = epage[t0 + min((int)threadIdx.x, n - 1)];
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int it = (int)threadIdx.x + u * kFusedThreads;
      if (it < NO * n) sh.kold[it % n][it / n] = kv[u];
    }
    if ((int)threadIdx.x < n) sh.eold[threadIdx.x] = ev;
    __syncthreads();
    if (w == 0) {
      if (lane < NQ) {
        for (int tt = 0; tt < n; ++tt) {
          const uint4 o8 = sh.kold[tt][lane >> 1];
          const uint32_t x = (lane & 1) ? o8.z : o8.x, y = (lane & 1) ? o8.w : o8.y;
          a0 += (double)bf16_lo(x);
          a1 += (double)bf16_hi(x);
          a2 += (double)bf16_lo(y);
          a3 += (double)bf16_hi(y);
        }
      } else if (lane == NQ) {
        for (int tt = 0; tt < n; ++tt) ae += (double)sh.eold[tt];
      }
    }
    __syncthreads();  // the staging buffers are reused by the next pass
  }
  if (w != 0) return;
  const double inv_n = 1.0 / (double)(r - lo + 1);
  const int s = i * nsub + j;
  if (lane < NQ) {
    const uint2 k_quad = reinterpret_cast<const uint2*>(kn)[lane];
    a0 += (double)bf16_lo(k_quad.x);
    a1 += (double)bf16_hi(k_quad.x);
    a2 += (double)bf16_lo(k_quad.y);
    a3 += (double)bf16_hi(k_quad.y);
    f4 o;
    o.x = (float)(a0 * inv_n);
    o.y = (float)(a1 * inv_n);
    o.z = (float)(a2 * inv_n);
    o.w = (float)(a3 * inv_n);
    reinterpret_cast<f4*>(a.k_summary)[((int64_t)bh * NQ + lane) * CS + s] = o;
    sh.knew[lane] = o;
  } else if (lane == NQ) {
    ae += (double)e_new;
    const float em = (float)(ae * inv_n);
    a.e_summary[(int64_t)bh * CS + s] = em;
    sh.enew = em;
    sh.have_new = 1;
  }
  // the new token itself (the older ones were read above)
  if (lane < NO) reinterpret_cast<uint4*>(kpage)[lane * bs + r] = reinterpret_cast<const uint4*>(kn)[lane];
#pragma unroll
  for (int jj = 0; jj < VL; ++jj) vpage[((r / 8) * D + lane + jj * kWave) * 8 + r % 8] = vn[lane + jj * kWave];
  if (lane == 0) epage[r] = e_new;
}

// Whether the lead workgroup loads its summaries before its append (with the
// lookups; one memory round trip fewer on the launch's critical path): where
// a lane's slice is at most 8 quads and the kernel still fits 8 waves per
// SIMD (64 VGPRs) without spills with them live across the append (not the
// QKV variants, whose eviction head needs more registers).
template <int D, int L, bool ROPE, bool QKV>
constexpr bool kEarlySummary() {
  return !ROPE && !QKV && D / 4 / L <= 8;
}

// L lanes per sub-block (see score_kernel).  ROPE: packed table, scoring
// only, nsub >= 4.  QKV: the appended token and the query from the fused
// projection rows.
template <int D, int L, bool ROPE = false, bool QKV = false>
__global__ __launch_bounds__(kFusedThreads)
__attribute__((amdgpu_waves_per_eu(kEarlySummary<D, L, ROPE, QKV>() || ROPE ? 8 : 1))) void append_score_kernel(const FusedArgs a) {
  constexpr int NQ = D / 4;
  constexpr int QL = NQ / L;
  constexpr int SPW = kWave / L;
  constexpr int SPG = SPW * (kFusedThreads / kWave);
  __shared__ FusedSmem<D, ROPE ? 1 : kStageTok> sh;
  __shared__ RopeSmem<D, ROPE> rsh;
  const Table& t = a.t;
  const int bh = blockIdx.y;
  const int Hkv = t.Hkv;
  const int b = bh / Hkv, h = bh % Hkv;
  const int G = a.Hq / Hkv;
  const int bs = a.bs, ss = a.ss, nsub = bs / ss;
  const int MB = t.max_blocks, CS = MB * nsub, cap = MB * bs;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;

  // the new token's k and v, and the group's query: separate inputs, or
  // slices of the sequence's projection row
  const uint16_t* kn;
  const uint16_t* vn;
  const uint16_t* qbase;
  if constexpr (QKV) {
    const uint16_t* row = a.qkv + (int64_t)b * (a.Hq + 2 * Hkv) * D;
    qbase = row + (int64_t)h * G * D;
    kn = row + ((int64_t)a.Hq + h) * D;
    vn = row + ((int64_t)a.Hq + Hkv + h) * D;
  } else {
    qbase = a.q + ((int64_t)b * a.Hq + (int64_t)h * G) * D;
    kn = a.k_new + (int64_t)bh * D;
    vn = a.v_new + (int64_t)bh * D;
  }
  const bool want_append = !ROPE && (QKV || a.k_new != nullptr);  // the RoPE variant only scores
  const int c = (int)gridDim.x - 1 - (int)blockIdx.x;  // chunks last to first
  const int s0 = c * SPG;
  // Issued together, before any of them is needed: the length, the pages of
  // this chunk's blocks (with an append: one lane per block in every wave,
  // so the append needs no dependent table lookup), the group's query.
  const int raw = a.seq_in[b];
  const int bpc = SPG / nsub;  // blocks per chunk (<= 64)
  int64_t spec_page = -1;
  if (want_append && lane < bpc && c * bpc + lane < MB) {
    uint32_t doc;
    spec_page = page_of_any(t, bh, c * bpc + lane, doc);
  }
  const int dq = threadIdx.x < D ? threadIdx.x : 0;
  const uint16_t* qh = qbase + dq;
  uint16_t qraw[16];
#pragma unroll
  for (int g = 0; g < 16; ++g) qraw[g] = qh[(int64_t)min(g, G - 1) * D];

  const bool append = want_append && raw >= 0 && raw < cap;
  const int T = min(max(append ? raw + 1 : raw, 0), cap);
  const int nb = (T + bs - 1) / bs;
  const int sT = append ? (raw / bs) * nsub + (raw % bs) / ss : -1;  // the new token's sub-block
  const bool work = s0 < nb * nsub;
  const bool lead = append && s0 <= sT && sT < s0 + SPG;
  if (threadIdx.x == 0) {
    sh.have_new = 0;
    if (blockIdx.x == 0 && h == 0 && want_append) {
      if (!append) flag_error(t.err);
      a.seq_out[b] = append ? raw + 1 : raw;
    }
  }

  // this lane's slice of its sub-block's summary row
  const int s = s0 + w * SPW + lane % SPW;
  const int part = lane / SPW;
  f4 v[QL];
  float ev = 0.f;
  auto load_summary = [&]() {
    const f4* p = reinterpret_cast<const f4*>(a.k_summary) + (int64_t)bh * NQ * CS + min(s, CS - 1) +
                  (int64_t)(part * QL) * CS;
#pragma unroll
    for (int u = 0; u < QL; ++u) v[u] = __builtin_nontemporal_load(p + (int64_t)u * CS);
    ev = a.e_summary[(int64_t)bh * CS + min(s, CS - 1)];
  };
  // every other workgroup loads right away; the lead too where its
  // registers allow (its append then adds one memory round trip, the older
  // tokens, instead of two), else after the append
  constexpr bool early = kEarlySummary<D, L, ROPE, QKV>();
  // (the RoPE variant loads after its rotations, so that the loaded rows are
  // not held across them)
  if (!ROPE && work && (early || !lead)) load_summary();
  if (threadIdx.x < D) {
    double acc = 0;
#pragma unroll
    for (int g = 0; g < 16; ++g) acc += g < G ? (double)bf16_to_f32(qraw[g]) : 0.0;
    sh.qbar[threadIdx.x] = acc / (double)G;
  }
  __syncthreads();  // have_new cleared before the append sets it
  if constexpr (QKV) {  // the split query, for the decode (one workgroup per pair)
    if (blockIdx.x == 0) {
      for (int u = threadIdx.x; u < G * D / 8; u += kFusedThreads)
        reinterpret_cast<uint4*>(a.q_out + ((int64_t)b * a.Hq + (int64_t)h * G) * D)[u] =
            reinterpret_cast<const uint4*>(qbase)[u];
    }
  }
  if (lead) {  // the page of the new token's block, from this wave's lookups
    const int idx = raw / bs - c * bpc;
    const int64_t page = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(spec_page >> 32), idx) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane((int)spec_page, idx));
    float e_new;
    if constexpr (QKV) {  // the eviction head: w_h . v in float64, one rounding
      const float* wh = a.w_evict + (int64_t)h * D;
      double acc = 0;
#pragma unroll
      for (int jd = 0; jd < D / kWave; ++jd) {
        const int d = lane + jd * kWave;
        acc = fma((double)bf16_to_f32(vn[d]), (double)wh[d], acc);
      }
      acc = xor_reduce<1, kWave>(acc, [](double x, double y) { return x + y; });
      e_new = (float)acc;
    } else {
      e_new = a.e_new[bh];
    }
    append_token(a, sh, bh, raw, page, kn, vn, e_new);
    if constexpr (!early) load_summary();
  }
  __syncthreads();  // qbar, and the append's summary

  if constexpr (ROPE) {
    // The rotated mean query once per distinct document among this
    // workgroup's blocks (documents span many blocks: usually one), wave r %
    // 4 turning document r, shared through LDS; `work` is uniform over the
    // workgroup, so every thread meets the barriers.
    constexpr int NBG = kFusedThreads / kWave * kRopeBlocksPerWave;  // >= SPG / nsub
    const int nbg = SPG / nsub;
    const int blkg = s0 / nsub;
    if (work && w == 0) {
      uint32_t docw = 0xffffffffu;  // past the table: a document of its own
      if (lane < nbg && blkg + lane < MB) (void)page_of<NOSA_TABLE_PACKED_ROPE>(t, bh, blkg + lane, docw);
      if (lane < NBG) rsh.docb[lane] = docw;
      wave_lds_sync();
      const bool first = lane < nbg && (lane == 0 || rsh.docb[lane - 1] != docw);
      const uint64_t starts = __ballot(first);
      if (lane < nbg) rsh.didx[lane] = __popcll(starts & ((2ull << lane) - 1ull)) - 1;
      if (first) rsh.dst[__popcll(starts & ((1ull << lane) - 1ull))] = docw;
      if (lane == 0) rsh.ndoc = __popcll(starts);
    }
    __syncthreads();
    if (work) {
      const int ndoc = rsh.ndoc;
      const int64_t n = a.q_pos[b];
      for (int r = w; r < ndoc; r += kFusedThreads / kWave) {  // (uniform per wave)
        if (lane < D / 2) {
          const double theta = pow(a.rope_base, -2.0 * (double)lane / (double)D);
          const int64_t st = (int64_t)rsh.dst[r] * bs;
          double sv, cv;
          sincos((double)(n - st) * theta, &sv, &cv);
          const double x1 = sh.qbar[lane], x2 = sh.qbar[lane + D / 2];
          rsh.rq[r][lane] = x1 * cv - x2 * sv;
          rsh.rq[r][lane + D / 2] = x2 * cv + x1 * sv;
        }
      }
      load_summary();
    }
    __syncthreads();
  }

  if (work) {
    if (lead && s == sT && sh.have_new) {  // this step's summary of the new token's sub-block
#pragma unroll
      for (int u = 0; u < QL; ++u) v[u] = sh.knew[part * QL + u];
      ev = sh.enew;
    }
    const int i = s / nsub, j = s % nsub;
    const bool valid = i < nb && i * bs + j * ss < T;
    double a0 = 0, a1 = 0, a2 = 0, a3 = 0;
    if constexpr (ROPE) {
      const double* rq = rsh.rq[rsh.didx[(w * SPW + lane % SPW) / nsub]];
#pragma unroll
      for (int u = 0; u < QL; ++u) {
        const int d = 4 * (part * QL + u);
        a0 = fma((double)v[u].x, rq[d + 0], a0);
        a1 = fma((double)v[u].y, rq[d + 1], a1);
        a2 = fma((double)v[u].z, rq[d + 2], a2);
        a3 = fma((double)v[u].w, rq[d + 3], a3);
      }
    } else {
#pragma unroll
      for (int u = 0; u < QL; ++u) {
        const int d = 4 * (part * QL + u);
        a0 = fma((double)v[u].x, sh.qbar[d + 0], a0);
        a1 = fma((double)v[u].y, sh.qbar[d + 1], a1);
        a2 = fma((double)v[u].z, sh.qbar[d + 2], a2);
        a3 = fma((double)v[u].w, sh.qbar[d + 3], a3);
      }
    }
    double dot = (a0 + a1) + (a2 + a3);
    dot = xor_reduce<SPW, kWave>(dot, [](double x, double y) { return x + y; });  // the L slices
    if (!valid) dot = -INFINITY;
    float ek = valid ? ev : -INFINITY;
    dot = xor_reduce_below(dot, nsub, [](double x, double y) { return fmax(x, y); });
    ek = xor_reduce_below(ek, nsub, [](float x, float y) { return fmaxf(x, y); });
    if (valid && part == 0 && j == 0) {
      a.score_q[(int64_t)bh * MB + i] = (float)(dot / sqrt((double)D));
      a.score_e[(int64_t)bh * MB + i] = ek;
    }
  }
}

hipError_t launch_append_score_qkv(const nosa_dims& d, const nosa_kv& kv, const uint16_t* qkv, const float* w_evict,
                                   const int32_t* seq_lens_in, int32_t* seq_lens_out, float* k_summary,
                                   float* e_summary, uint16_t* q_out, float* score_q, float* score_e,
                                   hipStream_t stream) {
  FusedArgs a = {};
  a.t = make_table(d, kv);
  a.Hq = d.n_q_heads;
  a.bs = d.block_size;
  a.ss = d.sub_block;
  a.k_pages = kv.k_pages;
  a.v_pages = kv.v_pages;
  a.e_pages = kv.e_pages;
  a.seq_in = seq_lens_in;
  a.seq_out = seq_lens_out;
  a.k_summary = k_summary;
  a.e_summary = e_summary;
  a.score_q = score_q;
  a.score_e = score_e;
  a.qkv = qkv;
  a.w_evict = w_evict;
  a.q_out = q_out;
  const int nsub = d.block_size / d.sub_block;
  const int CS = d.max_blocks * nsub;
  const int L = nsub <= 16 ? 4 : (nsub <= 32 ? 2 : 1);
  const int spg = (kWave / L) * (kFusedThreads / kWave);
  const dim3 grid((CS + spg - 1) / spg, d.batch * d.n_kv_heads);
#define NOSA_APPEND_SCORE_QKV(DD, LL) \
  append_score_kernel<DD, LL, false, true><<<grid, kFusedThreads, 0, stream>>>(a)
  if (d.head_dim == 128) {
    if (L == 4) NOSA_APPEND_SCORE_QKV(128, 4);
    else if (L == 2) NOSA_APPEND_SCORE_QKV(128, 2);
    else NOSA_APPEND_SCORE_QKV(128, 1);
  } else {
    if (L == 4) NOSA_APPEND_SCORE_QKV(64, 4);
    else if (L == 2) NOSA_APPEND_SCORE_QKV(64, 2);
    else NOSA_APPEND_SCORE_QKV(64, 1);
  }
#undef NOSA_APPEND_SCORE_QKV
  return hipGetLastError();
}

hipError_t launch_append_score(const nosa_dims& d, const nosa_kv& kv, const uint16_t* k_new,
                               const uint16_t* v_new, const float* e_new, const int32_t* seq_lens_in,
                               int32_t* seq_lens_out, float* k_summary, float* e_summary, const uint16_t* q,
                               float* score_q, float* score_e, hipStream_t stream) {
  FusedArgs a = {};
  a.t = make_table(d, kv);
  a.Hq = d.n_q_heads;
  a.bs = d.block_size;
  a.ss = d.sub_block;
  a.k_new = k_new;
  a.v_new = v_new;
  a.e_new = e_new;
  a.k_pages = kv.k_pages;
  a.v_pages = kv.v_pages;
  a.e_pages = kv.e_pages;
  a.seq_in = seq_lens_in;
  a.seq_out = seq_lens_out;
  a.k_summary = k_summary;
  a.e_summary = e_summary;
  a.q = q;
  a.score_q = score_q;
  a.score_e = score_e;
  a.q_pos = kv.q_pos;
  a.rope_base = (double)kv.rope_base;
  const int nsub = d.block_size / d.sub_block;
  const int CS = d.max_blocks * nsub;
  const int L = nsub <= 16 ? 4 : (nsub <= 32 ? 2 : 1);  // as score_kernel
  const int spg = (kWave / L) * (kFusedThreads / kWave);
  const dim3 grid((CS + spg - 1) / spg, d.batch * d.n_kv_heads);
#define NOSA_APPEND_SCORE(DD, LL) append_score_kernel<DD, LL><<<grid, kFusedThreads, 0, stream>>>(a)
  if (kv.kind == NOSA_TABLE_PACKED_ROPE) {  // scoring only, nsub in [4, 16] (L == 4)
    if (d.head_dim == 128)
      append_score_kernel<128, 4, true><<<grid, kFusedThreads, 0, stream>>>(a);
    else
      append_score_kernel<64, 4, true><<<grid, kFusedThreads, 0, stream>>>(a);
    return hipGetLastError();
  }
  if (d.head_dim == 128) {
    if (L == 4) NOSA_APPEND_SCORE(128, 4);
    else if (L == 2) NOSA_APPEND_SCORE(128, 2);
    else NOSA_APPEND_SCORE(128, 1);
  } else {
    if (L == 4) NOSA_APPEND_SCORE(64, 4);
    else if (L == 2) NOSA_APPEND_SCORE(64, 2);
    else NOSA_APPEND_SCORE(64, 1);
  }
#undef NOSA_APPEND_SCORE
  return hipGetLastError();
}

}  // namespace nosa
