// Split-K flash decoding over the selected pages, and the combine.
//
// Novita AI blog "How KV sparsity achieves 1.5x acceleration for vLLM",
// Key techniques, 2. Attention modifications: FlashAttention walks the KV
// blocks once, keeping O, the running row max and the running sum l, and
// divides O by l at the end; the row max and l are cheap to return with O.
// Here the pass runs only over the pages of the selected blocks (NOSA
// summary, Methodology 1, dual selection; Spin summary 2.B, per-head
// pages; 2.C, two-level index), split into contiguous chunks of the
// selected list whose (o, m, l) partials the combine merges.
//
// Deferred RoPE (LazyAttention summary, Technical implementation,
// 2. Decoding; Mathematical equivalence): stored keys carry only their
// in-document rotation; the query is rotated by (query position - document
// start) once per document, inside the loop, and the (page, document start)
// pair comes from one packed 32-bit word, so the kernel still reads only K
// and V.
//
// gfx950 mapping.  Workgroup = 4 waves = one (b, h) pair x one split.  The
// work unit is a 64-token tile of a selected block; wave w takes tiles w,
// w+4, ... and keeps its own online-softmax state, and the four states are
// merged through LDS at the end.  Both products run on the matrix cores
// (v_mfma_f32_16x16x32_bf16) with the GQA group packed block-diagonally:
//   q . k:  A = keys (16 token rows x 32 k slots), B = the group's query,
//           non-zero only where a column's token set owns the k slots, so
//           every output column is a real (token set, head) pair and the
//           softmax runs on useful lanes only.  The query stays in
//           registers for the whole workgroup.
//   P . V:  A = V^T (16 dims x 32 token slots), B = the tile's bf16
//           probabilities (block diagonal again, one LDS round trip per
//           tile); per-set partial outputs are summed once at the end.
// Page layouts make every operand a single 16-byte load per lane:
//   K page [D/8][bs][8] -> A rows of q.k (runs of 16 tokens x 16 bytes);
//   V page [bs/8][D][8] -> A rows of P.V (8 tokens of one dim per load).
// The step is HBM-bound (4 bytes of K+V per token-dim); the matrix cores keep
// the arithmetic and operand broadcasts off the vector ALUs and out of the
// register file, which is what lets two waves per SIMD stay resident.  The
// query is exact bf16 and accumulation is fp32; probabilities enter P.V as
// bf16 while l sums the fp32 values.  With deferred RoPE the rotated query
// is split into bf16 hi + lo parts that fill spare head columns of the same
// MFMA (|error| ~ 2^-16 relative).
//
// Softmax score step (Novita page, 2. Attention modifications: with the
// returned row max and l, p = exp(q.k - rowmax) / l is each key's softmax
// score, summed row-wise into a sparsification score).  With MASS the wave
// also stores, per tile and head, the sum of the tile's fp32 probabilities
// and the running max they are relative to; the workgroup that completes the
// combine turns them into each selected block's softmax mass per query
// head, mass = sum over the block's tiles of l_t 2^(m_t - M) / L, with the
// final M and L.  K is not read again.
//
// ALiBi (LazyAttention summary, generalisation to other relative position
// schemes): keys carry no position, and each score gets -slope_j (n - t)
// for key position t and query position n = T - 1, added in the tile loop
// from the tile's first position; nothing else changes.

#include <mutex>

#include "nosa_launch.hpp"
#include "nosa_select_impl.hpp"

namespace nosa {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kTile = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeArgs {
  Table t;
  int Hq, bs, P, sel_cap;
  // splits per workgroup (1, or 2 on the plain variant: see split_group)
  int S;
  float scale_log2;  // sm_scale * log2(e): scores kept in log2 units
  float rope_base;
  const uint16_t* q;
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  const int32_t* sel;
  const int32_t* sel_count;
  const int32_t* seq_lens;
  const int32_t* q_pos;
  float* part_o;
  float* part_m;
  float* part_l;
  // fused combine (all null for the split-only call)
  int32_t* counters;  // [B*Hkv], zero between calls
  float* o;
  float* m;
  float* l;
  // fused selection (select variants only): every workgroup of a pair makes
  // the pair's selection; split 0 writes it, the new bitmap and the swap
  // lists out
  const float* score_q;
  const float* score_e;
  int k_e, k_q;
  const uint32_t* ev_in;
  uint32_t* ev_out;
  int32_t* sel_w;
  int32_t* sel_count_w;
  SwapArgs sw;
  // softmax score step (MASS variants only)
  float* tile_stats;  // [B*Hkv][sel_cap * bs/64][G][2]: tile sum of p, running max (log2 units)
  float* mass;        // [B][Hq][sel_cap]
  // ALiBi (ALIBI variants only)
  const float* alibi;  // [Hq] slopes
};

// The select variants hold SR elements per select thread: SR = 4 covers
// max_blocks <= 1024, SR = 9 max_blocks <= 2304 (a 256K context of
// 128-token blocks plus appended tokens).  A lane of a wave holds bitmap
// words lane and, with SR = 9, lane + 64.
constexpr int kDecSelMaxBlocks = 9 * kSelThreads;
static_assert(kDecSelMaxBlocks == NOSA_SELECT_DECODE_MAX_BLOCKS, "the C-ABI limit is the kernels' own");

// LDS of the fused selection (SR > 0: elements per select thread).
template <int SR>
struct DecodeSelSmem {
  SelShared sel;
  int32_t list[SR * kSelThreads];  // the blocks to decode
  int32_t total;                   // tiles of the list, once published (-1 before)
};
// spins of a wave waiting for the query part's tiles (about 60 ns each; far
// beyond any selection's duration): past it the wave flags an error and stops
constexpr int kPublishSpinLimit = 1 << 20;
// the one-wave query selection's duration in tile times of one wave, for
// sharing the query part's tiles out (one tile: ~4-6 us per wave at one
// wave per SIMD).  Measured best: 1 for its 16 rows (SR = 4; 0-2 within
// noise), 6-8 for its 36 rows (SR = 9, 2050 blocks).
template <int SR>
constexpr int kSelectTiles = SR <= 4 ? 1 : 7;
template <>
struct DecodeSelSmem<0> {};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Page data is read once per step: non-temporal loads stream it past the
// caches (on gfx950 these sustain far more HBM bandwidth than ordinary
// loads for this access pattern).
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// D(16x16) += A(16x32) . B(32x16), bf16 inputs, fp32 accumulation.  Lane
// l = 16 q + r supplies A row r and B column r for the eight k slots of lane
// group q, and receives D rows 4q .. 4q+3 of column r.
__device__ __forceinline__ floatx4 mfma_bf16(const uint4& a, const uint4& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Columns of one MFMA: GE head slots per token set, 16 / GE token sets.  A
// set's k slots are LPS lane groups, and the query operand is zero outside
// its own set's slots (block diagonal), so one MFMA scores 16 * (16 / GE)
// tokens against GE head slots with no padded output.  With deferred RoPE
// head slots G .. 2G-1 carry the low bf16 part of the rotated query.
template <int D, int G, bool ROPE>
struct DecodeShape {
  static constexpr int GR = ROPE ? 2 * G : G;  // head slots carrying data
  static constexpr int GE = GR <= 8 ? 8 : 16;  // head slots per set
  static constexpr int NC = 16 / GE;           // token sets per MFMA
  static constexpr int LPS = 4 / NC;           // lane groups per set
  static constexpr int TPM = 16 * NC;          // tokens per q.k MFMA
  static constexpr int TH = kTile / TPM;       // token slices per tile
  static constexpr int DPM = 8 * LPS;          // dims per q.k MFMA
  static constexpr int NDS = D / DPM;          // q.k MFMAs per slice
  static constexpr int NDT = D / 16;           // P.V dim tiles
  static_assert(GR <= 16, "at most 16 head slots");
};

template <int D, int G, bool ROPE>
struct DecodeSmem {
  int32_t last;
  uint16_t p[kDecWaves][G][kTile];  // bf16 probabilities of the tile, per wave
  float qf[ROPE ? G : 1][ROPE ? D : 1];
  uint16_t qrot[ROPE ? kDecWaves : 1][ROPE ? 2 * G : 1][ROPE ? D : 8];  // rotated query, bf16 hi / lo rows
  float mw[kDecWaves][G];
  float lw[kDecWaves][G];
  float ow[kDecWaves][G][D];
};

// Split partials cross workgroups in the fused decode + combine: written
// with store_coherent, read back with load_f32<true>, and ordered by the
// wait-then-count arrival at the end of decode_kernel.

// Merge of the P split partials of one output row at dim d [NOVITA, 2.
// Attention modifications]: M = max of the non-empty splits' row maxima,
// weights l_p * exp(m_p - M), O = sum_p w_p O_p / sum_p w_p.  The first
// PRE splits are loaded together (clamped, branch-free) so P <= PRE costs
// one memory round trip; later splits are loaded one at a time.  Callers
// take PRE = 8 up to eight splits and 16 above (merge_splits_p).  Thread (row, d); the thread with d == 0 also
// writes the row's m and l.  COHERENT: the partials come from other
// workgroups of the same launch (device-scope loads).
template <bool COHERENT, int PRE>
__device__ __forceinline__ void merge_splits(int P, int D, int64_t row, int d, const float* __restrict__ part_o,
                                             const float* __restrict__ part_m, const float* __restrict__ part_l,
                                             float* __restrict__ o, float* __restrict__ m, float* __restrict__ l) {
  const float* pm = part_m + row * P;
  const float* pl = part_l + row * P;
  const float* po = part_o + row * P * D + d;
  float mv[PRE], lv[PRE], ov[PRE];
#pragma unroll
  for (int j = 0; j < PRE; ++j) {
    const int k = min(j, P - 1);
    mv[j] = load_f32<COHERENT>(pm + k);
    lv[j] = load_f32<COHERENT>(pl + k);
    ov[j] = load_f32<COHERENT>(po + (int64_t)k * D);
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < PRE; ++j)
    if (j < P && lv[j] > 0.f) M = fmaxf(M, mv[j]);
  for (int k = PRE; k < P; ++k) {
    const float lk = load_f32<COHERENT>(pl + k), mk = load_f32<COHERENT>(pm + k);
    if (lk > 0.f) M = fmaxf(M, mk);
  }
  float L = 0.f, O = 0.f;
#pragma unroll
  for (int j = 0; j < PRE; ++j) {
    if (j < P && lv[j] > 0.f) {
      const float wj = lv[j] * expf(mv[j] - M);
      L += wj;
      O += wj * ov[j];
    }
  }
  for (int k = PRE; k < P; ++k) {
    const float lk = load_f32<COHERENT>(pl + k), mk = load_f32<COHERENT>(pm + k);
    if (lk > 0.f) {
      const float wk = lk * expf(mk - M);
      L += wk;
      O += wk * load_f32<COHERENT>(po + (int64_t)k * D);
    }
  }
  o[row * D + d] = L > 0.f ? O / L : 0.f;
  if (d == 0) {
    m[row] = L > 0.f ? M : -INFINITY;
    l[row] = L;
  }
}

// merge_splits with the prefetch depth for P: the same operations in the
// same order either way, so the result does not depend on it.
template <bool COHERENT>
__device__ __forceinline__ void merge_splits_p(int P, int D, int64_t row, int d, const float* __restrict__ part_o,
                                               const float* __restrict__ part_m, const float* __restrict__ part_l,
                                               float* __restrict__ o, float* __restrict__ m, float* __restrict__ l) {
  if (P > 8)
    merge_splits<COHERENT, 16>(P, D, row, d, part_o, part_m, part_l, o, m, l);
  else
    merge_splits<COHERENT, 8>(P, D, row, d, part_o, part_m, part_l, o, m, l);
}

// merge_splits for P == 1 with the split's values already in registers:
// the same operations in the same order, so the result is bit-identical.
__device__ __forceinline__ void merge_one(float pm, float pl, float po, int64_t row, int d, int D,
                                          float* __restrict__ o, float* __restrict__ m, float* __restrict__ l) {
  float M = -INFINITY;
  if (pl > 0.f) M = fmaxf(M, pm);
  float L = 0.f, O = 0.f;
  if (pl > 0.f) {
    const float w = pl * expf(pm - M);
    L += w;
    O += w * po;
  }
  o[row * D + d] = L > 0.f ? O / L : 0.f;
  if (d == 0) {
    m[row] = L > 0.f ? M : -INFINITY;
    l[row] = L;
  }
}

// Softmax mass of every selected block of pair bh for query head g of the
// group, given the final row max M2 (log2 units) and sum L of that head:
// the sum over the block's tiles that hold tokens of l_t 2^(m_t - M2) / L.
// Entries n .. sel_cap-1 receive 0.  Threads of the workgroup split the
// (head, block) pairs; the tile statistics are read with device-scope
// loads (they may come from other workgroups of the launch).
template <int G, int KIND>
__device__ __forceinline__ void finish_mass(const Table& t, int bh, int b, int h, int Hq, int bs, int sel_cap, int n,
                                            int T, const int32_t* list, const float* tile_stats, const float* M2,
                                            const float* L, float* mass) {
  const int tpb = bs / kTile;
  const int nb = (T + bs - 1) / bs;
  for (int x = threadIdx.x; x < G * sel_cap; x += kDecThreads) {
    const int g = x / sel_cap, j = x % sel_cap;
    float acc = 0.f;
    if (j < n && L[g] > 0.f) {
      const int i = list[j];
      uint32_t docb;
      if (i >= 0 && i < nb && page_of<KIND>(t, bh, i, docb) >= 0) {
        for (int sub = 0; sub < tpb; ++sub) {
          if (T - (i * bs + sub * kTile) <= 0) break;  // no tokens from here on
          const float* st = tile_stats + (((int64_t)bh * sel_cap * tpb + (int64_t)j * tpb + sub) * G + g) * 2;
          acc += load_f32<true>(st) * exp2f(load_f32<true>(st + 1) - M2[g]);
        }
        acc /= L[g];
      }
    }
    mass[((int64_t)b * Hq + (int64_t)h * G + g) * sel_cap + j] = acc;
  }
}

// SR > 0: the select variant (SR elements per thread of the selection,
// covering max_blocks <= SR * kSelThreads).  MASS: the softmax score step
// (SR == 0 with the fused combine only).  ALIBI: ALiBi biases (SR == 0).
//
// Select variant.  On most steps the eviction part has nothing to choose:
// the blocks it has never dropped number at most k_e (a new one appears only
// when the context crosses a block boundary), so it keeps all of them, and
// they are known from the incoming bitmap at launch [NOSA summary,
// Methodology 1, locality guarantee: the eviction part changes only by
// dropping].  Each workgroup then lists those blocks at once; wave 0 makes
// the query part alone (select_query_wave) while waves 1-3 already decode
// eviction-part tiles, so the selection no longer holds the HBM idle.  The
// query part's size, min(k_q, nb - n_e), is known at launch too, so the
// work is shared out by a fixed rule: split p takes the p-th of P equal
// shares (whole blocks) of the eviction part and of the query part; in the
// workgroup, waves 1-3 take the share's eviction tiles round-robin, wave 0
// the first Q0 of its query tiles (Q0 balances its selection time) and
// waves 1-3 the rest.  The schedule depends on the inputs only, so results
// are reproducible bit for bit.  Otherwise (a new block competes) all four
// waves make the whole selection first (select_pair), split p takes the
// p-th contiguous chunk of the ascending list, and the waves take its
// tiles round-robin.  Against the separate calls, the tiles' visiting
// order differs, and on the fast path with several splits which blocks
// each split's partial covers; the merged output is the same attention.
template <int D, int G, int KIND, int SR, bool MASS = false, bool ALIBI = false>
__global__ __launch_bounds__(kDecThreads, SR > 0 ? 1 : 2) void decode_kernel(const DecodeArgs a) {
  constexpr bool ROPE = KIND == NOSA_TABLE_PACKED_ROPE;
  using S = DecodeShape<D, G, ROPE>;
  constexpr int GE = S::GE, LPS = S::LPS, TPM = S::TPM, TH = S::TH, NDS = S::NDS, NDT = S::NDT;
  __shared__ DecodeSmem<D, G, ROPE> sh;
  __shared__ DecodeSelSmem<SR> ssh;
  static_assert(SR == 0 || kDecThreads == kSelThreads, "the selection runs on the whole workgroup");
  static_assert(!(MASS && SR > 0) && !(ALIBI && SR > 0), "select variants decode plain scores");

  const int bh = blockIdx.x, p = blockIdx.y;
  const int Hkv = a.t.Hkv;
  const int b = bh / Hkv, h = bh % Hkv;
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  // splits per workgroup and waves per split (the select, mass and ALiBi
  // variants take one split per workgroup)
  const int spw = SR > 0 || MASS || ALIBI ? 1 : a.S;
  const int wps = kDecWaves / spw;
  const int w_s = __builtin_amdgcn_readfirstlane(w);  // the wave index, in a scalar register
  const int lq = lane >> 4, lr = lane & 15;    // lane group, row/column
  const int set_q = lq / LPS, dsub = lq % LPS;  // k slots of this lane group
  const int cset = lr / GE, cg = lr % GE;       // column: token set, head slot
  const bool qcol = cset == set_q && cg < S::GR; // query operand non-zero
  const bool real = cg < G;                     // column of a real head

  const int T = min(max(a.seq_lens[b], 0), a.t.max_blocks * a.bs);
  const int nb = (T + a.bs - 1) / a.bs;
  const int tpb = a.bs / kTile;
  const uint16_t* qg = a.q + ((int64_t)b * a.Hq + (int64_t)h * G) * D;  // heads h*G.. are contiguous

  // query operand of q.k, one 16-byte slice per d-step.  The select variant
  // parks the query in LDS during the selection (its loads go out before the
  // selection's inputs, and it holds no registers meanwhile).
  uint4 qreg[NDS];
  double theta = 0.0;
  int64_t qpos = 0;
  __shared__ uint4 qstage[SR > 0 && !ROPE ? G * D / 8 : 1];
  auto query_from = [&](const uint4* src) {
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const int o = ds * LPS + dsub;
      qreg[ds] = qcol ? src[(cg * D + 8 * o) / 8] : make_uint4(0, 0, 0, 0);
    }
  };
  if constexpr (SR > 0) {
    if constexpr (ROPE) {  // the query itself is parked in sh.qf during the selection
      if (lane < D / 2) theta = pow((double)a.rope_base, -2.0 * (double)lane / (double)D);
      qpos = a.q_pos[b];
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) qreg[ds] = make_uint4(0, 0, 0, 0);
    }
  } else if constexpr (!ROPE) {
    query_from(reinterpret_cast<const uint4*>(qg));
  } else {
    for (int k = threadIdx.x; k < G * D; k += kDecThreads) sh.qf[k / D][k % D] = bf16_to_f32(qg[k]);
    if (lane < D / 2) theta = pow((double)a.rope_base, -2.0 * (double)lane / (double)D);
    qpos = a.q_pos[b];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qreg[ds] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  }

  // K as the A operand: row lr of token set set_q, octet ds*LPS + dsub;
  // V^T as the A operand of P.V: dim 16 dt + lr, tokens 32 ks + 8 lq .. +8
  auto k_ptr = [&](int64_t page, int sub) {
    return reinterpret_cast<const uint4*>(a.k_pages + page * (int64_t)a.bs * D) + sub * kTile + 16 * set_q + lr +
           (int64_t)dsub * a.bs;
  };
  auto v_ptr = [&](int64_t page, int sub) {
    return reinterpret_cast<const uint4*>(a.v_pages + page * (int64_t)a.bs * D) + (sub * 8 + lq) * D + lr;
  };
  uint4 kr[TH][NDS];
  uint4 vr[2][NDT];
  auto load_tile = [&](int64_t page, int sub) {
    const uint4* kpg = k_ptr(page, sub);
#pragma unroll
    for (int th = 0; th < TH; ++th)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) kr[th][ds] = load_stream(kpg + (int64_t)ds * LPS * a.bs + th * TPM);
    const uint4* vpg = v_ptr(page, sub);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vr[ks][dt] = load_stream(vpg + ks * 4 * D + dt * 16);
  };

  int n = 0;
  const int32_t* selp = a.sel + (int64_t)bh * a.sel_cap;  // global list (SR == 0)
  // Tile c of this workgroup is the 64-token slice c % tpb of list entry
  // lbase + c / tpb; wave w takes tiles w, w + 4, ... of its split's chunk,
  // except on the fast path of the select variants (tile_of below).
  int lbase = 0, ntiles = 0;
  // fast path of the select variants: list tiles [0, e_t) are the eviction
  // part's, from e_t on the query part's; this split's share is le tiles
  // from e_lo and lqt tiles from e_t + q_lo, and wave 0 takes the first q0
  // of the latter
  bool fast = false;
  int e_t = 0, e_lo = 0, le = 0, q_lo = 0, lqt = 0, q0 = 0;
  const float* sq_row = a.score_q + (int64_t)bh * a.t.max_blocks;
  const float* se_row = a.score_e + (int64_t)bh * a.t.max_blocks;
  if constexpr (SR > 0) {
    const bool lead = p == 0;
    const int words = (a.t.max_blocks + 31) / 32;  // <= 2 * kWave
    // the incoming bitmap (words lane and lane + 64; missing words read as
    // all dropped) and each thread's piece of the query, loaded first
    const uint32_t* evp = a.ev_in + (int64_t)bh * words;
    const uint32_t evw = lane < words ? evp[lane] : 0xffffffffu;
    const uint32_t evw2 = SR > 8 && lane + kWave < words ? evp[lane + kWave] : 0xffffffffu;
    constexpr int kQPieces = G * D / 8;
    static_assert(kQPieces <= kDecThreads, "one query piece per thread");
    const bool has_piece = (int)threadIdx.x < kQPieces;
    uint4 qp = make_uint4(0, 0, 0, 0);
    if (has_piece) qp = reinterpret_cast<const uint4*>(qg)[threadIdx.x];
    // the query into LDS: bf16 octets to stage (or, with deferred RoPE, as
    // floats in sh.qf, rotated per document in the tile loop)
    auto park_query = [&]() {
      if (!has_piece) return;
      if constexpr (ROPE) {
        const int k0 = 8 * (int)threadIdx.x;  // elements k0 .. k0 + 7 of the G x D query
        const uint32_t wv[4] = {qp.x, qp.y, qp.z, qp.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sh.qf[(k0 + 2 * e) / D][(k0 + 2 * e) % D] = bf16_lo(wv[e]);
          sh.qf[(k0 + 2 * e + 1) / D][(k0 + 2 * e + 1) % D] = bf16_hi(wv[e]);
        }
      } else {
        qstage[threadIdx.x] = qp;
      }
    };
    // only split 0 writes the selection's outputs (the swap lists too)
    SwapArgs sw = a.sw;  // a copy (see select_pair)
    if (!lead) sw.load = nullptr;
    // wave 0's inputs of the one-wave query selection go out at once too,
    // before the other waves load pages (wasted if the step takes the
    // four-wave selection: 4 * SR KB)
    constexpr int RQ = SR * kSelThreads / kWave;
    QueryWaveInputs<RQ> qin;
    if (w == 0) load_query_wave<RQ>(qin, bh, a.t.max_blocks, sq_row, a.sel_cap, sw);
    // the blocks below nb the eviction part has never dropped: bits of
    // word lane (blocks from base), then of word lane + 64 (from base2)
    auto never_dropped = [&](uint32_t word, int from) -> uint32_t {
      return from >= nb ? 0u : (nb - from >= 32 ? ~word : ~word & ((1u << (nb - from)) - 1u));
    };
    const int base = lane * 32, base2 = base + 32 * kWave;
    const uint32_t z = never_dropped(evw, base);
    const uint32_t z2 = SR > 8 ? never_dropped(evw2, base2) : 0u;
    const int cz = __popc(z), cz2 = __popc(z2);
    const int incl = wave_scan_incl(cz);
    const int n_lo = __builtin_amdgcn_readlane(incl, kWave - 1);  // in words 0 .. 63
    int incl2 = 0, n_cand = n_lo;
    if constexpr (SR > 8) {
      incl2 = wave_scan_incl(cz2);
      n_cand += __builtin_amdgcn_readlane(incl2, kWave - 1);
    }
    fast = n_cand <= a.k_e;
    if (fast) {
      // the eviction part keeps them all: wave 0 lists them (ascending), then
      // makes the query part while the other waves decode its share of them
      if (w == 0) {
        uint32_t zz = z;
        for (int j = incl - cz; zz != 0u; ++j) {
          ssh.list[j] = base + __ffs(zz) - 1;
          zz &= zz - 1u;
        }
        if constexpr (SR > 8) {
          zz = z2;
          for (int j = n_lo + incl2 - cz2; zz != 0u; ++j) {
            ssh.list[j] = base2 + __ffs(zz) - 1;
            zz &= zz - 1u;
          }
        }
      }
      if (threadIdx.x == 0) ssh.total = -1;
      const int n_q = max(0, min(a.k_q, nb - n_cand));
      const int e0 = (int)((int64_t)p * n_cand / a.P), e1 = (int)((int64_t)(p + 1) * n_cand / a.P);
      const int qa = (int)((int64_t)p * n_q / a.P), qb = (int)((int64_t)(p + 1) * n_q / a.P);
      e_t = n_cand * tpb;
      e_lo = e0 * tpb;
      le = (e1 - e0) * tpb;
      q_lo = qa * tpb;
      lqt = (qb - qa) * tpb;
      q0 = min(max((le + lqt - 3 * kSelectTiles<SR>) / kDecWaves, 0), lqt);
      park_query();
      __syncthreads();  // the eviction part's list, the query
      if constexpr (!ROPE) query_from(qstage);
      if (w == 0) {
        n = select_query_wave<RQ>(qin, bh, nb, a.t.max_blocks, a.k_q, evw, evw2, n_cand, lead ? a.ev_out : nullptr,
                                  lead ? a.sel_w + (int64_t)bh * a.sel_cap : nullptr, a.sel_cap,
                                  lead ? a.sel_count_w + bh : nullptr, sw, ssh.sel.hist[0], ssh.sel.pick_bm,
                                  ssh.sel.prev_bm, ssh.list + n_cand);
        // the query part's tiles follow the eviction part's (list written above)
        if (lane == 0) __hip_atomic_store(&ssh.total, n * tpb, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    } else {
      // the whole selection, by all four waves, into LDS; split 0 also
      // writes the outputs.  The query waits in LDS meanwhile.
      auto after_loads = [&]() { park_query(); };
      n = select_pair<SR, true>(ssh.sel, bh, T, a.bs, a.t.max_blocks, sq_row, se_row, a.k_e, a.k_q,
                                a.ev_in + (int64_t)bh * words, lead ? a.ev_out + (int64_t)bh * words : nullptr,
                                ssh.list, a.sel_cap, nullptr, sw, after_loads);
      const int cc = (n + a.P - 1) / a.P;
      const int j0 = min(p * cc, n), j1 = min(j0 + cc, n);
      lbase = j0;
      ntiles = (j1 - j0) * tpb;
      __syncthreads();  // the list, the query
      if constexpr (!ROPE) query_from(qstage);
      if (lead) {
        for (int k = threadIdx.x; k < n; k += kDecThreads) a.sel_w[(int64_t)bh * a.sel_cap + k] = ssh.list[k];
        if (threadIdx.x == 0) a.sel_count_w[bh] = n;
      }
    }
  } else {
    // this wave's split: workgroup p holds splits p spw .. p spw + spw - 1,
    // with wps = kDecWaves / spw waves on each
    n = min(max(a.sel_count[bh], 0), a.sel_cap);
    const int cc = (n + a.P - 1) / a.P;
    const int pw = p * spw + w_s / wps;
    const int j0 = min(pw * cc, n), j1 = min(j0 + cc, n);
    lbase = j0;
    ntiles = (j1 - j0) * tpb;
  }
  uint32_t cur_doc = 0xffffffffu;

  float m_run = -INFINITY, l_run = 0.f;  // for head slot cg, log2 units
  // ALiBi slope of head slot cg in log2 units, and the query position
  const float slope = ALIBI && real ? a.alibi[h * G + cg] * kLog2e : 0.f;
  const int qn = T - 1;
  floatx4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Tile j of this wave's schedule (-1: none left).  Round-robin over the
  // four waves, except on the fast path (see the kernel's comment).
  auto tile_of = [&](int j) -> int {
    if (!fast) {
      const int x = w_s % wps + wps * j;
      return x < ntiles ? x : -1;
    }
    // position x in this split's share: eviction tiles [0, le), query [le, le + lqt)
    int x;
    if (w == 0) {
      x = j < q0 ? le + j : le + lqt;
    } else {
      const int ne = le > w - 1 ? (le - w + 3) / 3 : 0;  // eviction-part tiles of this wave
      x = j < ne ? w - 1 + 3 * j : le + q0 + w - 1 + 3 * (j - ne);
    }
    if (x >= le + lqt) return -1;
    return x < le ? e_lo + x : e_t + q_lo + (x - le);
  };
  // Waves 1-3 wait for wave 0 to publish the query part's tiles before the
  // first of them (bounded: past the limit the wave flags an error and
  // takes no more tiles).
  bool published = !fast || w == 0;
  auto await_query_part = [&]() -> bool {
    if constexpr (SR > 0) {
      for (int spin = 0; !published; ++spin) {
        published = __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                        &ssh.total, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) >= 0;
        if (published) break;
        if (spin >= kPublishSpinLimit) {
          if (lane == 0) flag_error(a.t.err);
          return false;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    return true;
  };

  // The wave's next tile with data, from position j of its schedule on:
  // its page, token count, document, slice and first position; entries the
  // table cannot resolve are skipped and flagged.  Returns the schedule
  // position after it (jn) and the tile, or kNone when there is none.
  constexpr int kNone = INT_MAX;
  int jn = 0;
  auto next_tile = [&](int j, int64_t& page, int& ntok, uint32_t& docb, int& sub, int& pos0) -> int {
    for (;; ++j) {
      const int kf = tile_of(j);
      if (kf < 0) return kNone;
      if (kf >= e_t && !await_query_part()) return kNone;
      jn = j + 1;
      // the LDS list is read by name (LDS instructions): through a generic
      // pointer every read would also wait for the in-flight tile loads
      int i;
      if constexpr (SR > 0)
        i = ssh.list[lbase + kf / tpb];
      else
        i = selp[lbase + kf / tpb];
      sub = kf % tpb;
      if (i < 0 || i >= nb) {
        if (lane == 0) flag_error(a.t.err);
        continue;
      }
      page = page_of<KIND>(a.t, bh, i, docb);
      if (page < 0) {
        if (lane == 0) flag_error(a.t.err);
        continue;
      }
      if constexpr (ALIBI) pos0 = i * a.bs + sub * kTile;
      ntok = min(kTile, T - (i * a.bs + sub * kTile));
      if (ntok > 0) return kf;
    }
  };

  int64_t page = 0;
  int ntok = 0, sub = 0, pos0 = 0;
  uint32_t docb = 0;
  int k = next_tile(0, page, ntok, docb, sub, pos0);  // the current tile
  if (k != kNone) load_tile(page, sub);

  // Software pipeline: once q.k has consumed this tile's keys the key
  // registers receive the next tile's keys, and once P.V has consumed the
  // values they receive the next values, so every wave keeps a tile of
  // loads in flight while it computes.
  while (k != kNone) {
    int64_t npage = 0;
    int nntok = 0, nsub = 0, npos0 = 0;
    uint32_t ndocb = 0;
    const int nk = next_tile(jn, npage, nntok, ndocb, nsub, npos0);

    // Slots past the end hold stale page data.  A row of the q.k MFMA mixes
    // tokens of every token set (the query is zero outside a set's slots),
    // and 0 * NaN would leak into valid scores, so zero those keys.
    if (ntok < kTile) {
#pragma unroll
      for (int th = 0; th < TH; ++th)
        if (th * TPM + 16 * set_q + lr >= ntok)
#pragma unroll
          for (int ds = 0; ds < NDS; ++ds) kr[th][ds] = make_uint4(0, 0, 0, 0);
    }

    if constexpr (ROPE) {
      if (docb != cur_doc) {  // new document: query rotated by n - start
        cur_doc = docb;
        if (lane < D / 2) {
          double sv, cv;
          sincos((double)(qpos - (int64_t)docb * a.bs) * theta, &sv, &cv);
          // pair (lane, lane + D/2): first half x1 c - x2 s, second x2 c + x1 s;
          // bf16 hi part in rows 0..G-1, lo part in rows G..2G-1
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const double x1 = sh.qf[g][lane], x2 = sh.qf[g][lane + D / 2];
            const float r1 = (float)(x1 * cv - x2 * sv);
            const float r2 = (float)(x2 * cv + x1 * sv);
            const uint16_t h1 = f32_to_bf16(r1), h2 = f32_to_bf16(r2);
            sh.qrot[w][g][lane] = h1;
            sh.qrot[w][g][lane + D / 2] = h2;
            sh.qrot[w][G + g][lane] = f32_to_bf16(r1 - bf16_to_f32(h1));
            sh.qrot[w][G + g][lane + D / 2] = f32_to_bf16(r2 - bf16_to_f32(h2));
          }
        }
        wave_lds_sync();
        const int slot = qcol ? cg : 0;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const uint4 v = *reinterpret_cast<const uint4*>(&sh.qrot[w][slot][8 * (ds * LPS + dsub)]);
          qreg[ds] = qcol ? v : make_uint4(0, 0, 0, 0);
        }
      }
    }

    // scores: slice th, rows 4 lq + e of token set cset, head slot cg
    float sv[TH][4];
#pragma unroll
    for (int th = 0; th < TH; ++th) {
      floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) acc = mfma_bf16(kr[th][ds], qreg[ds], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = acc[e];
        if constexpr (ROPE) x += lane_xor<G>(x);  // hi + lo parts
        const int tok = th * TPM + 16 * cset + 4 * lq + e;
        if constexpr (ALIBI)
          sv[th][e] = tok < ntok ? x * a.scale_log2 - slope * (float)(qn - (pos0 + tok)) : -INFINITY;
        else
          sv[th][e] = tok < ntok ? x * a.scale_log2 : -INFINITY;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (nk != kNone) {  // prefetch the next tile's keys
      const uint4* kpg = k_ptr(npage, nsub);
#pragma unroll
      for (int th = 0; th < TH; ++th)
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) kr[th][ds] = load_stream(kpg + (int64_t)ds * LPS * a.bs + th * TPM);
    }

    // tile max per head slot: lanes sharing cg
    float mx = -INFINITY;
#pragma unroll
    for (int th = 0; th < TH; ++th)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sv[th][e]);
    mx = xor_reduce<GE, kWave>(mx, [](float x, float y) { return fmaxf(x, y); });
    const float mn = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - mn);
    m_run = mn;
    float psum = 0.f;
#pragma unroll
    for (int th = 0; th < TH; ++th) {
      uint32_t pw[2];
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float p0 = exp2f(sv[th][e] - mn), p1 = exp2f(sv[th][e + 1] - mn);
        psum += p0 + p1;
        pw[e / 2] = (uint32_t)f32_to_bf16(p0) | ((uint32_t)f32_to_bf16(p1) << 16);
      }
      if (real)
        *reinterpret_cast<uint2*>(&sh.p[w][cg][th * TPM + 16 * cset + 4 * lq]) = make_uint2(pw[0], pw[1]);
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
    if constexpr (MASS) {  // the tile's probability sum per head slot
      const float tsum = xor_reduce<GE, kWave>(psum, [](float x, float y) { return x + y; });
      if (real && cset == 0 && lq == 0) {
        float* st = a.tile_stats + (((int64_t)bh * a.sel_cap * tpb + (int64_t)lbase * tpb + k) * G + cg) * 2;
        store_coherent(st, tsum);
        store_coherent(st + 1, mn);
      }
    }

    // tokens past the end hold stale page data: zero their V entries
    if (ntok < kTile) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int nv = min(max(ntok - (32 * ks + 8 * lq), 0), 8);
        uint32_t mk[4];
#pragma unroll
        for (int jd = 0; jd < 4; ++jd)
          mk[jd] = (2 * jd < nv ? 0x0000ffffu : 0u) | (2 * jd + 1 < nv ? 0xffff0000u : 0u);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          vr[ks][dt].x &= mk[0];
          vr[ks][dt].y &= mk[1];
          vr[ks][dt].z &= mk[2];
          vr[ks][dt].w &= mk[3];
        }
      }
    }
    wave_lds_sync();

    // O^T(dims x head slots) += V^T . P, P block diagonal over token sets
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 pv = *reinterpret_cast<const uint4*>(&sh.p[w][real ? cg : 0][32 * ks + 8 * lq]);
      const bool on = real && cset == set_q;
      const uint4 pb = on ? pv : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] = mfma_bf16(vr[ks][dt], pb, oacc[dt]);
    }
    wave_lds_sync();
    __builtin_amdgcn_sched_barrier(0);
    if (nk != kNone) {  // prefetch the next tile's values
      const uint4* vpg = v_ptr(npage, nsub);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vr[ks][dt] = load_stream(vpg + ks * 4 * D + dt * 16);
    }
    k = nk;
    page = npage;
    ntok = nntok;
    sub = nsub;
    docb = ndocb;
    if constexpr (ALIBI) pos0 = npos0;
  }

  // per-wave totals: sum the token sets of each head slot, then the lanes
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      oacc[dt][e] = xor_reduce<GE, 16>(oacc[dt][e], [](float x, float y) { return x + y; });
  float lsum = l_run;
  lsum = xor_reduce<GE, kWave>(lsum, [](float x, float y) { return x + y; });
  if (real && cset == 0) {
    if (lq == 0) {
      sh.mw[w][cg] = m_run;
      sh.lw[w][cg] = lsum;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) sh.ow[w][cg][16 * dt + 4 * lq + e] = oacc[dt][e];
  }
  __syncthreads();

  // each split's partial: the merge of its waves' totals
  for (int k = threadIdx.x; k < spw * G * D; k += kDecThreads) {
    const int sp = k / (G * D), g = (k / D) % G, d = k % D;
    const int w0 = sp * wps, w1 = w0 + wps;
    float M = -INFINITY;
    for (int ww = w0; ww < w1; ++ww)
      if (sh.lw[ww][g] > 0.f) M = fmaxf(M, sh.mw[ww][g]);
    float L = 0.f, O = 0.f;
    for (int ww = w0; ww < w1; ++ww) {
      if (sh.lw[ww][g] > 0.f) {
        const float f = exp2f(sh.mw[ww][g] - M);
        L += sh.lw[ww][g] * f;
        O += sh.ow[ww][g][d] * f;
      }
    }
    const int64_t row = ((int64_t)b * a.Hq + (int64_t)h * G + g) * a.P + p * spw + sp;
    const float po = L > 0.f ? O / L : 0.f, pm = L > 0.f ? M * kLn2 : -INFINITY;
    store_coherent(a.part_o + row * D + d, po);
    if (d == 0) {
      store_coherent(a.part_m + row, pm);
      store_coherent(a.part_l + row, L);
    }
    if (a.o != nullptr && a.P == 1) {  // fused combine of a single split, in registers
      const int64_t orow = (int64_t)b * a.Hq + (int64_t)h * G + g;
      merge_one(pm, L, po, orow, d, D, a.o, a.m, a.l);
    }
  }

  if constexpr (MASS) {
    if (a.P == 1) {  // the final M and L are this workgroup's own merge
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();  // every wave's tile statistics
      __shared__ float fm[G], fl[G];
      if (threadIdx.x < G) {
        const int g = threadIdx.x;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww)
          if (sh.lw[ww][g] > 0.f) M = fmaxf(M, sh.mw[ww][g]);
        float L = 0.f;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww)
          if (sh.lw[ww][g] > 0.f) L += sh.lw[ww][g] * exp2f(sh.mw[ww][g] - M);
        fm[g] = M;
        fl[g] = L;
      }
      __syncthreads();
      finish_mass<G, KIND>(a.t, bh, b, h, a.Hq, a.bs, a.sel_cap, n, T, selp, a.tile_stats, fm, fl, a.mass);
      return;
    }
  }
  if (a.counters == nullptr || a.P == 1) return;
  // Fused combine: the last workgroup of this (b, h) to finish merges the P
  // partials.  Every wave waits for its device-scope partial stores to
  // complete, then one thread counts the workgroup's arrival; the last
  // arrival reads the partials back with device-scope loads.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (threadIdx.x == 0) sh.last = atomicAdd(&a.counters[bh], spw) == a.P - spw;
  __syncthreads();
  if (!sh.last) return;
  for (int k = threadIdx.x; k < G * D; k += kDecThreads) {
    const int g = k / D, d = k % D;
    const int64_t row = (int64_t)b * a.Hq + (int64_t)h * G + g;
    if constexpr (SR > 0)  // (up to four splits by default)
      merge_splits<true, 8>(a.P, D, row, d, a.part_o, a.part_m, a.part_l, a.o, a.m, a.l);
    else
      merge_splits_p<true>(a.P, D, row, d, a.part_o, a.part_m, a.part_l, a.o, a.m, a.l);
  }
  if constexpr (MASS) {  // final M (log2 units) and L of each head from the partials
    __shared__ float fm[G], fl[G];
    if (threadIdx.x < G) {
      const int64_t row = ((int64_t)b * a.Hq + (int64_t)h * G + threadIdx.x) * a.P;
      float M = -INFINITY;
      for (int q = 0; q < a.P; ++q)
        if (load_f32<true>(a.part_l + row + q) > 0.f) M = fmaxf(M, load_f32<true>(a.part_m + row + q) * kLog2e);
      float L = 0.f;
      for (int q = 0; q < a.P; ++q) {
        const float lq = load_f32<true>(a.part_l + row + q);
        if (lq > 0.f) L += lq * exp2f(load_f32<true>(a.part_m + row + q) * kLog2e - M);
      }
      fm[threadIdx.x] = M;
      fl[threadIdx.x] = L;
    }
    __syncthreads();
    finish_mass<G, KIND>(a.t, bh, b, h, a.Hq, a.bs, a.sel_cap, n, T, selp, a.tile_stats, fm, fl, a.mass);
  }
  if (threadIdx.x == 0) a.counters[bh] = 0;  // ready for the next call
}

// One workgroup per (b, query head), thread per dim; the same merge as the
// fused tail of decode_kernel.
__global__ void combine_kernel(int P, int D, const float* __restrict__ part_o, const float* __restrict__ part_m,
                               const float* __restrict__ part_l, float* __restrict__ o, float* __restrict__ m,
                               float* __restrict__ l) {
  merge_splits_p<false>(P, D, blockIdx.x, threadIdx.x, part_o, part_m, part_l, o, m, l);
}

// The select variants: SR = 4 up to 1024 blocks, SR = 9 up to 2304.
template <int D, int G, int SR>
static void launch_select_dg(dim3 grid, const DecodeArgs& a, int kind, hipStream_t stream) {
  switch (kind) {
    case NOSA_TABLE_FLAT:
      decode_kernel<D, G, NOSA_TABLE_FLAT, SR><<<grid, kDecThreads, 0, stream>>>(a);
      break;
    case NOSA_TABLE_TWO_LEVEL:
      decode_kernel<D, G, NOSA_TABLE_TWO_LEVEL, SR><<<grid, kDecThreads, 0, stream>>>(a);
      break;
    default:
      if constexpr (G <= 8) decode_kernel<D, G, NOSA_TABLE_PACKED_ROPE, SR><<<grid, kDecThreads, 0, stream>>>(a);
      break;
  }
}

template <int D, int G>
static void launch_decode_dg(dim3 grid, const DecodeArgs& a, int kind, bool select, hipStream_t stream) {
  if (a.alibi != nullptr) {  // ALiBi: flat and two-level tables
    if (kind == NOSA_TABLE_FLAT)
      decode_kernel<D, G, NOSA_TABLE_FLAT, 0, false, true><<<grid, kDecThreads, 0, stream>>>(a);
    else
      decode_kernel<D, G, NOSA_TABLE_TWO_LEVEL, 0, false, true><<<grid, kDecThreads, 0, stream>>>(a);
    return;
  }
  if (a.mass != nullptr) {  // the softmax score step: flat and two-level tables
    if (kind == NOSA_TABLE_FLAT)
      decode_kernel<D, G, NOSA_TABLE_FLAT, 0, true><<<grid, kDecThreads, 0, stream>>>(a);
    else
      decode_kernel<D, G, NOSA_TABLE_TWO_LEVEL, 0, true><<<grid, kDecThreads, 0, stream>>>(a);
    return;
  }
  if (select) {  // max_blocks <= kDecSelMaxBlocks
    if (a.t.max_blocks <= 4 * kSelThreads)
      launch_select_dg<D, G, 4>(grid, a, kind, stream);
    else
      launch_select_dg<D, G, 9>(grid, a, kind, stream);
    return;
  }
  switch (kind) {
    case NOSA_TABLE_FLAT:
      decode_kernel<D, G, NOSA_TABLE_FLAT, 0><<<grid, kDecThreads, 0, stream>>>(a);
      break;
    case NOSA_TABLE_TWO_LEVEL:
      decode_kernel<D, G, NOSA_TABLE_TWO_LEVEL, 0><<<grid, kDecThreads, 0, stream>>>(a);
      break;
    default:
      if constexpr (G <= 8) decode_kernel<D, G, NOSA_TABLE_PACKED_ROPE, 0><<<grid, kDecThreads, 0, stream>>>(a);
      break;
  }
}

template <int D>
static void launch_decode_d(dim3 grid, const DecodeArgs& a, int G, int kind, bool select, hipStream_t stream) {
  switch (G) {
    case 1: launch_decode_dg<D, 1>(grid, a, kind, select, stream); break;
    case 2: launch_decode_dg<D, 2>(grid, a, kind, select, stream); break;
    case 4: launch_decode_dg<D, 4>(grid, a, kind, select, stream); break;
    case 8: launch_decode_dg<D, 8>(grid, a, kind, select, stream); break;
    default: launch_decode_dg<D, 16>(grid, a, kind, select, stream); break;
  }
}

static DecodeArgs decode_args(const nosa_dims& d, const uint16_t* q, const nosa_kv& kv, const int32_t* sel,
                              const int32_t* sel_count, int32_t sel_cap, const int32_t* seq_lens, int32_t num_splits,
                              float sm_scale, float* part_o, float* part_m, float* part_l, int32_t* counters,
                              float* o, float* m, float* l) {
  DecodeArgs a = {};
  a.t = make_table(d, kv);
  a.Hq = d.n_q_heads;
  a.bs = d.block_size;
  a.P = num_splits;
  a.S = 1;
  a.sel_cap = sel_cap;
  a.scale_log2 = sm_scale * kLog2e;
  a.rope_base = kv.rope_base;
  a.q = q;
  a.k_pages = kv.k_pages;
  a.v_pages = kv.v_pages;
  a.sel = sel;
  a.sel_count = sel_count;
  a.seq_lens = seq_lens;
  a.q_pos = kv.q_pos;
  a.part_o = part_o;
  a.part_m = part_m;
  a.part_l = part_l;
  a.counters = counters;
  a.o = o;
  a.m = m;
  a.l = l;
  return a;
}

// Splits per workgroup of the plain decode.  Short splits (at most four
// 64-token tiles per wave) make short workgroups whose start-up and first
// loads are a large share of their time; a workgroup then takes two adjacent
// splits, two waves on each, so each wave streams twice the tiles.  Every
// split's partial is still its own (the merge of its waves), and the combine
// merges all P of them.  Kept to one where halving the grid would leave CUs
// without a workgroup, and on the select, mass and ALiBi variants.
constexpr int kSplitGroupMinWorkgroups = 256;

static int split_group(const nosa_dims& d, const DecodeArgs& a, bool select) {
  if (select || a.mass != nullptr || a.alibi != nullptr || a.P % 2 != 0) return 1;
  const int64_t tiles_per_split = (int64_t)((a.sel_cap + a.P - 1) / a.P) * (a.bs / kTile);
  const int64_t groups = (int64_t)d.batch * d.n_kv_heads * (a.P / 2);
  return tiles_per_split <= 4 * kDecWaves && groups >= kSplitGroupMinWorkgroups ? 2 : 1;
}

static hipError_t launch_decode_args(const nosa_dims& d, const DecodeArgs& args, int kind, bool select,
                                     hipStream_t stream) {
  DecodeArgs a = args;
  a.S = split_group(d, a, select);
  const dim3 grid(d.batch * d.n_kv_heads, a.P / a.S);
  const int G = d.n_q_heads / d.n_kv_heads;
  if (d.head_dim == 128)
    launch_decode_d<128>(grid, a, G, kind, select, stream);
  else
    launch_decode_d<64>(grid, a, G, kind, select, stream);
  return hipGetLastError();
}

hipError_t launch_decode(const nosa_dims& d, const uint16_t* q, const nosa_kv& kv,
                         const int32_t* sel, const int32_t* sel_count, int32_t sel_cap,
                         const int32_t* seq_lens, int32_t num_splits, float sm_scale,
                         float* part_o, float* part_m, float* part_l, int32_t* counters, float* o,
                         float* m, float* l, hipStream_t stream) {
  const DecodeArgs a = decode_args(d, q, kv, sel, sel_count, sel_cap, seq_lens, num_splits, sm_scale, part_o,
                                   part_m, part_l, counters, o, m, l);
  return launch_decode_args(d, a, kv.kind, false, stream);
}

hipError_t launch_select_decode(const nosa_dims& d, const uint16_t* q, const nosa_kv& kv, const float* score_q,
                                const float* score_e, const int32_t* seq_lens, int32_t k_e, int32_t k_q,
                                const uint32_t* evicted_in, uint32_t* evicted_out, int32_t* sel, int32_t sel_cap,
                                int32_t* sel_count, const int32_t* prev, const int32_t* prev_count, int32_t* load,
                                int32_t* load_count, int32_t* evict, int32_t* evict_count, int32_t num_splits,
                                float sm_scale, float* part_o, float* part_m, float* part_l, int32_t* counters,
                                float* o, float* m, float* l, hipStream_t stream) {
  DecodeArgs a = decode_args(d, q, kv, nullptr, nullptr, sel_cap, seq_lens, num_splits, sm_scale, part_o, part_m,
                             part_l, counters, o, m, l);
  a.score_q = score_q;
  a.score_e = score_e;
  a.k_e = k_e;
  a.k_q = k_q;
  a.ev_in = evicted_in;
  a.ev_out = evicted_out;
  a.sel_w = sel;
  a.sel_count_w = sel_count;
  a.sw = SwapArgs{prev, prev_count, load, load_count, evict, evict_count};
  return launch_decode_args(d, a, kv.kind, true, stream);
}

// ---------------------------------------------------------------------------
// nosa_select_decode_noalloc: the workspaces of the fused select + decode (the
// split partials and the per-pair arrival counters of the cross-workgroup
// combine) in a fixed device array of the library instead of caller memory,
// for callers that cannot allocate.  Each GPU holds its own copy of the
// array; host code uses its device address, looked up once per device.  The
// counters must be zero at the start of a call: the loader zero-fills the
// array, set-up clears the counter region once more with a kernel (a memset
// node would misbehave in a captured graph), and every call leaves them
// zero.  Calls that overlap on one GPU share the array and race.
// ---------------------------------------------------------------------------

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;

__global__ void zero_words_kernel(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// Device address of this GPU's scratch array (set up on first use).
static hipError_t scratch_address(unsigned char** out, hipStream_t stream) {
  static std::mutex mu;
  static unsigned char* addr[kMaxScratchDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    unsigned char* base = static_cast<unsigned char*>(p);
    zero_words_kernel<<<64, 256, 0, stream>>>(reinterpret_cast<int32_t*>(base + kNoAllocCountersOffset),
                                              kNoAllocCountersBytes / 4);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    addr[dev] = base;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_select_decode_noalloc(const nosa_dims& d, const uint16_t* q, const nosa_kv& kv,
                                        const float* score_q, const float* score_e, const int32_t* seq_lens,
                                        int32_t k_e, int32_t k_q, const uint32_t* evicted_in, uint32_t* evicted_out,
                                        int32_t* sel, int32_t sel_cap, int32_t* sel_count, const int32_t* prev,
                                        const int32_t* prev_count, int32_t* load, int32_t* load_count,
                                        int32_t* evict, int32_t* evict_count, int32_t num_splits, float sm_scale,
                                        float* o, float* m, float* l, hipStream_t stream) {
  const NoAllocLayout lay = noalloc_layout(d, num_splits);
  if (lay.total > kNoAllocScratchBytes) return hipErrorInvalidValue;  // the C-ABI layer checks first
  unsigned char* base = nullptr;
  const hipError_t e = scratch_address(&base, stream);
  if (e != hipSuccess) return e;
  return launch_select_decode(d, q, kv, score_q, score_e, seq_lens, k_e, k_q, evicted_in, evicted_out, sel,
                              sel_cap, sel_count, prev, prev_count, load, load_count, evict, evict_count,
                              num_splits, sm_scale, reinterpret_cast<float*>(base + lay.part_o),
                              reinterpret_cast<float*>(base + lay.part_m), reinterpret_cast<float*>(base + lay.part_l),
                              reinterpret_cast<int32_t*>(base + kNoAllocCountersOffset), o, m, l, stream);
}

hipError_t launch_decode_mass(const nosa_dims& d, const uint16_t* q, const nosa_kv& kv, const int32_t* sel,
                              const int32_t* sel_count, int32_t sel_cap, const int32_t* seq_lens, int32_t num_splits,
                              float sm_scale, float* part_o, float* part_m, float* part_l, int32_t* counters, float* o,
                              float* m, float* l, float* tile_stats, float* mass, hipStream_t stream) {
  DecodeArgs a = decode_args(d, q, kv, sel, sel_count, sel_cap, seq_lens, num_splits, sm_scale, part_o, part_m,
                             part_l, counters, o, m, l);
  a.tile_stats = tile_stats;
  a.mass = mass;
  return launch_decode_args(d, a, kv.kind, false, stream);
}

hipError_t launch_decode_alibi(const nosa_dims& d, const uint16_t* q, const nosa_kv& kv, const int32_t* sel,
                               const int32_t* sel_count, int32_t sel_cap, const int32_t* seq_lens,
                               int32_t num_splits, float sm_scale, const float* alibi_slopes, float* part_o,
                               float* part_m, float* part_l, int32_t* counters, float* o, float* m, float* l,
                               hipStream_t stream) {
  DecodeArgs a = decode_args(d, q, kv, sel, sel_count, sel_cap, seq_lens, num_splits, sm_scale, part_o, part_m,
                             part_l, counters, o, m, l);
  a.alibi = alibi_slopes;
  return launch_decode_args(d, a, kv.kind, false, stream);
}

hipError_t launch_combine(const nosa_dims& d, int32_t num_splits, const float* part_o,
                          const float* part_m, const float* part_l, float* o, float* m, float* l,
                          hipStream_t stream) {
  combine_kernel<<<d.batch * d.n_q_heads, d.head_dim, 0, stream>>>(num_splits, d.head_dim, part_o, part_m,
                                                                    part_l, o, m, l);
  return hipGetLastError();
}

}  // namespace nosa
