// Prefill attention over reused documents with deferred RoPE.
//
// LazyAttention summary, Technical implementation, 1. Prefilling: cached KV
// blocks are loaded while the prompt is processed, and instead of rotating
// keys twice (back to position 0, then to their new position) the kernel
// applies a single relative rotation from the offset between the queries
// and the cached document; Mathematical equivalence: RoPE attention depends
// only on that offset.  Stored keys carry their in-document rotation, so
//   Rot(n) q . Rot(st) k_stored = Rot(n - st) q . k_stored
// for a query at position n and a document starting at st.  The relative
// rotation is applied to the query, once per (query column, document) --
// documents span many key tiles, so this is rarer than rotating every K
// tile -- and the keys stream from their pages untouched.
//
// gfx950 mapping.  Workgroup = 8 waves = one (b, KV head) and 128 query
// columns (a column is a (prompt position, head of the group) pair); wave w
// owns 16 columns.  Keys stream in 64-token tiles that all eight waves share
// through LDS (eight waves rather than four halve the tile loads per column;
// the register file holds two waves per SIMD, so one workgroup per CU).
// Tile t + 1 goes from memory straight into the next of three LDS buffers
// (global_load_lds, no registers and no LDS stores) while tile t is
// computed, and is waited for just before the one barrier per tile; the
// pages of a run of 512 tiles are looked up together into LDS beforehand, so
// no tile waits on a table lookup.  Workgroups are placed XCD-aware: the
// workgroups of one (b, KV head) run on one XCD, so its K and V stream from
// that XCD's L2 after the first reader.  Both products run on
// v_mfma_f32_16x16x32_bf16 as in the decode: S^T = K . Q^T with the key rows
// as the A operand straight from the K page layout, and O^T += V^T . P with
// V^T rows from the V page layout and the tile's bf16 probabilities as the B
// operand, moved from the S^T accumulator layout into the operand layout by
// lane swaps in registers.  Waves 4-7 run their P.V one tile late (from the
// third buffer), so that the two waves sharing a SIMD are in different
// phases rather than in step.  The rotated query is split into bf16 hi + lo
// parts (two MFMAs per chunk) so the rotation costs no precision beyond
// ~2^-16.  Online softmax per column in log2 units: the q.k accumulators
// start at minus a reference that trails the running max by at most 16
// (probabilities below 2^16), so the scores arrive shifted and only a tile
// that moves some column's max past that slack pays for a rescale; the exact
// max is kept beside it for the outputs.  The column sums come
// from the P.V product itself, with an all-ones operand in place of V^T.
// Causal mask t <= n; keys past the context are masked and their V entries
// zeroed (0 * stale NaN would leak through the MFMA).

#include <type_traits>

#include "nosa_device.hpp"
#include "nosa_launch.hpp"

namespace nosa {

constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfTile = 64;  // keys per tile
constexpr int kPfBufs = 3;   // K and V tile buffers
constexpr int kPfCols = 16;  // query columns per wave
constexpr int kPfXcds = 8;  // XCDs: consecutive workgroups go to consecutive XCDs
// s_waitcnt vmcnt(0) alone (expcnt and lgkmcnt at their maxima)
constexpr int kVmcntZero = 0x0F70;
constexpr float kPfLog2e = 1.4426950408889634f;
constexpr float kPfLn2 = 0.6931471805599453f;
constexpr float kPfShiftSlack = 16.f;  // log2 units

struct PrefillArgs {
  Table t;
  int Hq, bs, M;
  int n_pairs, n_chunks;  // (b, KV head) pairs and 128-column chunks per pair
  float scale_log2;
  double rope_base;
  const uint16_t* q;  // [B][M][Hq][D], unrotated
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  const int32_t* q_pos0;    // [B] position of the first prompt token
  const int32_t* seq_lens;  // [B]
  float* o;                 // [B][M][Hq][D]
  float* m;                 // [B][M][Hq]
  float* l;
};

template <int D>
struct PrefillShared {
  float cs[kPfBufs][D / 2][2];              // cos, sin of st * theta_k, per tile buffer
  int2 pt[kPfThreads];                      // (page, document start in blocks) of a run of tiles
};
// One K and one V tile buffer.  Each buffer is a __shared__ variable of its
// own, so the compiler can tell the direct loads into one buffer from the
// reads of the other and does not wait for those loads before the reads.
template <int D>
struct PrefillKTile {
  uint4 u[D / 8][kPfTile];  // page layout [D/8][64][8]
};
template <int D>
struct PrefillVTile {
  uint4 u[kPfTile / 8][D];  // page layout [64/8][D][8]
};
template <int B>
struct PfBuf {
  static constexpr int value = B;
};
template <int B, class X>
__device__ __forceinline__ X& pf_pick(X& x0, X& x1, X& x2) {
  if constexpr (B == 0)
    return x0;
  else if constexpr (B == 1)
    return x1;
  else
    return x2;
}

typedef __bf16 pf_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pf_floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ pf_floatx4 pf_mfma(const uint4& a, const uint4& b, const pf_floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pf_bf16x8, a), __builtin_bit_cast(pf_bf16x8, b),
                                                 c, 0, 0, 0);
}

typedef __bf16 pf_bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values as packed bf16, round to nearest even (one
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float x0, float x1) {
  const pf_bf16x2 v = {(__bf16)x0, (__bf16)x1};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x with the hardware's v_exp_f32 alone: results below 2^-126 flush to
// zero (probabilities that small are nothing beside the row's sum), where
// exp2f spends four more instructions on keeping them.
__device__ __forceinline__ float pf_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 rounded to bf16 (nearest even) and back.
__device__ __forceinline__ float round_bf16(float x) { return (float)(__bf16)x; }

// Packs 8 fp32 values as bf16.
__device__ __forceinline__ uint4 pack_bf16x8(const float* x) {
  return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                    pack_bf16x2(x[6], x[7]));
}

// Column lr of wave w: prompt row m0 + w * (16 / G) + lr / G, head lr % G.
template <int D, int G>
__global__ __launch_bounds__(kPfThreads, 1) void prefill_rope_kernel(const PrefillArgs a) {
  constexpr int NCH = D / 32;      // 32-dim chunks of q.k
  constexpr int NDT = D / 16;      // 16-dim tiles of P.V
  constexpr int PPW = kPfCols / G;  // prompt rows per wave
  constexpr int KU = (D / 8) * kPfTile / kPfThreads;  // K tile units per thread
  constexpr int VU = (kPfTile / 8) * D / kPfThreads;  // V tile units per thread
  static_assert(KU >= 1 && VU >= 1, "tile units per thread");
  static_assert(kPfCols % G == 0, "G divides 16");
  __shared__ PrefillShared<D> sh;
  __shared__ PrefillKTile<D> k0, k1, k2;
  __shared__ PrefillVTile<D> v0, v1, v2;

  const Table& t = a.t;
  // XCD-aware placement: workgroup i runs on XCD i % 8; the workgroups of
  // one XCD take consecutive (pair, chunk) slots, so a pair's chunks share
  // an L2.  Slots past the last return at once (the whole workgroup).
  const int total = a.n_pairs * a.n_chunks, per_xcd = (total + kPfXcds - 1) / kPfXcds;
  const int slot = (int)(blockIdx.x % kPfXcds) * per_xcd + (int)(blockIdx.x / kPfXcds);
  if (slot >= total) return;
  const int bh = slot / a.n_chunks, chunk = slot % a.n_chunks;
  const int Hkv = t.Hkv;
  const int b = bh / Hkv, h = bh % Hkv;
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lq = lane >> 4, lr = lane & 15;
  const int bs = a.bs;
  const int T = min(max(a.seq_lens[b], 0), t.max_blocks * bs);
  const int m0 = chunk * (kPfWaves * PPW);
  const int mi = m0 + w * PPW + lr / G;
  const int g = lr % G;
  const bool col_ok = mi < a.M;
  const int64_t p0 = a.q_pos0[b];
  const int64_t n = p0 + min(mi, a.M - 1);  // this column's position (idle columns: the last row)
  const int mlast = min(m0 + kPfWaves * PPW, a.M) - 1;
  const int64_t last_key = min(p0 + mlast, (int64_t)T - 1);
  const int ntile = last_key >= 0 ? (int)(last_key / kPfTile) + 1 : 0;

  // Rot(n) q for this lane's column and dims 32 c + 8 lq + e, in fp32
  // (float64 angles, once), times the score scale in log2 units: the
  // rotation is linear, so q.k then comes out in the softmax's units
  float qn[NCH][8];
  {
    const uint16_t* qp = a.q + (((int64_t)b * a.M + min(mi, a.M - 1)) * a.Hq + (int64_t)h * G + g) * D;
#pragma unroll
    for (int c = 0; c < NCH / 2; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 32 * c + 8 * lq + e;  // < D/2; partner d + D/2 in chunk c + NCH/2
        const double x1 = bf16_to_f32(qp[d]), x2 = bf16_to_f32(qp[d + D / 2]);
        const double th = pow(a.rope_base, -2.0 * (double)d / (double)D);
        double sv, cv;
        sincos((double)n * th, &sv, &cv);
        qn[c][e] = (float)((x1 * cv - x2 * sv) * (double)a.scale_log2);
        qn[c + NCH / 2][e] = (float)((x2 * cv + x1 * sv) * (double)a.scale_log2);
      }
    }
  }
  const double theta_k = threadIdx.x < D / 2 ? pow(a.rope_base, -2.0 * (double)threadIdx.x / (double)D) : 0.0;

  uint4 qhi[NCH], qlo[NCH];
  // Column lr's reference for the shifted scores (log2 units), and the
  // exact running max over this lane's keys (the column's is reduced at the
  // end).  The reference moves only when a key lies more than kPfShiftSlack
  // above it, so the probabilities stay below 2^kPfShiftSlack (far inside
  // fp32 and bf16 range) and most tiles that raise a column's max skip the
  // rescale; the exact max and the sum taken against it are what the column
  // returns.
  float m_run = -INFINITY;
  float m_hi = -INFINITY;
  pf_floatx4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = pf_floatx4{0.f, 0.f, 0.f, 0.f};
  // column lr's running sum of the bf16 probabilities, every element: the
  // P.V product with an all-ones A operand sums each column over the keys
  pf_floatx4 lacc = pf_floatx4{0.f, 0.f, 0.f, 0.f};
  const uint32_t one2 = 0x3F803F80u;  // bf16 (1, 1)
  const uint4 ones = make_uint4(one2, one2, one2, one2);

  // Page and document start of tiles [c kPfThreads, (c + 1) kPfThreads),
  // one tile per thread, into the LDS run table: one memory round trip per
  // kPfThreads tiles instead of a dependent lookup per tile.  An
  // unresolvable tile raises the error flag and gets page -1.
  auto resolve_run = [&](int c) {
    const int tile = c * kPfThreads + (int)threadIdx.x;
    int2 e = make_int2(-1, 0);
    if (tile < ntile) {
      uint32_t docb = 0;
      const int64_t pg = page_of<NOSA_TABLE_PACKED_ROPE>(t, bh, tile * kPfTile / bs, docb);
      if (pg < 0) flag_error(t.err);
      e = make_int2((int)pg, (int)docb);
    }
    sh.pt[threadIdx.x] = e;
  };
  // tile -> page and document start (tokens) from the run table; page < 0:
  // unresolvable
  auto tile_page = [&](int tile, int64_t& page, int64_t& st) {
    const int2 e = sh.pt[tile % kPfThreads];
    page = e.x;
    st = (int64_t)(uint32_t)e.y * bs;
  };
  // Tile `tile` of page `page` straight from memory into the tile buffers
  // kd, vd (global_load_lds: lane l of a wave writes the 16 bytes at the
  // wave's LDS base + 16 l, so the 64 units of one wave-instruction,
  // consecutive in the page layout, land consecutively); an unresolvable
  // tile is zero-filled.  The data is in LDS once this wave's vector-memory
  // count reaches zero.
  // This thread's units of a tile: K unit u = tid + 512 j is row u / 64 =
  // w + 8 j, key u % 64 = lane of the page's [D/8][bs][8] layout; V unit u
  // sits u units into the tile's slice of the [bs/8][D][8] layout.  The byte
  // offsets do not change from tile to tile; only the page base does.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  uint32_t koff[KU], voff[VU];
#pragma unroll
  for (int j = 0; j < KU; ++j) koff[j] = (uint32_t)(((wu + (kPfThreads / kPfTile) * j) * bs + lane) * 16);
#pragma unroll
  for (int j = 0; j < VU; ++j) voff[j] = (uint32_t)((threadIdx.x + j * kPfThreads) * 16);
  auto fetch_lds = [&](int tile, int64_t page, PrefillKTile<D>& kd, PrefillVTile<D>& vd) {
    const int sub = (tile * kPfTile % bs) / kPfTile;
    uint4* kdu = &kd.u[0][0] + kWave * wu;  // this wave's 64 units, then every 512
    uint4* vdu = &vd.u[0][0] + kWave * wu;
    if (page >= 0) {
      const char* kb =
          reinterpret_cast<const char*>(a.k_pages + page * (int64_t)bs * D) + (int64_t)sub * kPfTile * 16;
      const char* vb = reinterpret_cast<const char*>(a.v_pages + page * (int64_t)bs * D) + (int64_t)sub * 8 * D * 16;
      // (the source address goes in as a uint4 pointer: given a char
      // pointer, the host pass drops the kernel's launch stub without a word)
#pragma unroll
      for (int j = 0; j < KU; ++j)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(kb + koff[j]),
                                         (__attribute__((address_space(3))) void*)(kdu + j * kPfThreads), 16, 0, 0);
#pragma unroll
      for (int j = 0; j < VU; ++j)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(vb + voff[j]),
                                         (__attribute__((address_space(3))) void*)(vdu + j * kPfThreads), 16, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < KU; ++j) kdu[lane + j * kPfThreads] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < VU; ++j) vdu[lane + j * kPfThreads] = make_uint4(0, 0, 0, 0);
    }
  };
  // After the wait: V of keys past the context zeroed (0 * stale NaN would
  // leak through the MFMA), in the units this thread loaded; only a tile
  // that reaches past the context has any.
  auto mask_tail = [&](int tile, PrefillVTile<D>& vd) {
    const int key0 = tile * kPfTile;
    if (key0 + kPfTile <= T) return;  // (uniform)
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = threadIdx.x + j * kPfThreads;
      const int ko = u / D;
      const int nv = min(max(T - (key0 + 8 * ko), 0), 8);  // present keys of this unit
      if (nv < 8) {
        uint4 x = vd.u[ko][u % D];
        uint32_t mk[4];
#pragma unroll
        for (int jd = 0; jd < 4; ++jd)
          mk[jd] = (2 * jd < nv ? 0x0000ffffu : 0u) | (2 * jd + 1 < nv ? 0xffff0000u : 0u);
        x.x &= mk[0];
        x.y &= mk[1];
        x.z &= mk[2];
        x.w &= mk[3];
        vd.u[ko][u % D] = x;
      }
    }
  };
  // cos, sin of st * theta_k into table `buf` (threads < D/2)
  auto rotation_table = [&](int64_t st, int buf) {
    if (threadIdx.x < D / 2) {
      double sv, cv;
      sincos((double)st * theta_k, &sv, &cv);
      sh.cs[buf][threadIdx.x][0] = (float)cv;
      sh.cs[buf][threadIdx.x][1] = (float)sv;
    }
  };
  auto wait_loads = [] { __builtin_amdgcn_s_waitcnt(kVmcntZero); };

  // prologue: tile 0 in buffer 0 with its rotation table
  int64_t page = -1, st = 0;         // page and document start of the tile being loaded
  int64_t st_cur = -1, st_next = 0;  // document starts of tiles t and t + 1
  bool ok_next = false;              // tile t + 1 resolvable
  resolve_run(0);
  __syncthreads();
  if (ntile > 0) {
    tile_page(0, page, st);
    fetch_lds(0, page, k0, v0);
    rotation_table(st, 0);
    st_next = st;
    ok_next = page >= 0;
    wait_loads();
    mask_tail(0, v0);
  }
  __syncthreads();

  int64_t rot_st = -1;  // the document start qhi / qlo are rotated for

  // S^T for one tile: rows = keys 16 th + 4 lq + e, column lr.  Chunk-major
  // order: the four key slices' accumulators are independent, so
  // consecutive MFMAs do not wait on each other's results.  The accumulators
  // start at -ref, ref = the running max (0 before the column's first key),
  // so the scores come out relative to it.
  auto qk_tile = [&](PrefillKTile<D>& kc, pf_floatx4* acc) {
    const float ref = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int th = 0; th < 4; ++th) acc[th] = pf_floatx4{-ref, -ref, -ref, -ref};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      uint4 ka[4];
#pragma unroll
      for (int th = 0; th < 4; ++th) ka[th] = kc.u[4 * c + lq][16 * th + lr];
#pragma unroll
      for (int th = 0; th < 4; ++th) acc[th] = pf_mfma(ka[th], qhi[c], acc[th]);
#pragma unroll
      for (int th = 0; th < 4; ++th) acc[th] = pf_mfma(ka[th], qlo[c], acc[th]);
    }
  };
  // Online softmax of one tile's shifted scores: masks (only where `full` is
  // false), the running max, the rescale of the accumulators when some
  // column's max moved, and the bf16 probabilities in the P.V operand
  // layout (pb[ks] for keys 32 ks .. 32 ks + 31).
  auto softmax_tile = [&](const pf_floatx4* acc, int key0, bool tile_ok, bool full, uint4* pb) {
    const float ref = m_run == -INFINITY ? 0.f : m_run;
    float sv[4][4];
#pragma unroll
    for (int th = 0; th < 4; ++th)
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[th][e] = acc[th][e];
    if (!full) {  // (uniform) key 16 th + 4 lq + e is visible iff 16 th + e <= lim
      const int64_t lim64 = min((int64_t)T - 1, n) - (key0 + 4 * lq);
      const int lim = (int)max(min(lim64, (int64_t)kPfTile), (int64_t)-1) | -(int)!tile_ok;
#pragma unroll
      for (int th = 0; th < 4; ++th)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[th][e] = 16 * th + e <= lim ? sv[th][e] : -INFINITY;
    }
    // This lane's max over its 16 scores.  The exact max is kept per lane
    // (the column's is reduced once, at the end).  The reference moves when
    // a key lies more than the slack above it, or at the column's first
    // visible keys: a lane that sees either calls for the column maxima
    // (a cross-lane reduction), and only then (rare after the first tiles)
    // are the scores shifted by d and the accumulators scaled by 2^-d (by 0
    // at the first keys: they hold nothing yet).
    float mx = -INFINITY;
#pragma unroll
    for (int th = 0; th < 4; ++th)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sv[th][e]);
    m_hi = fmaxf(m_hi, ref + mx);
    const bool want = mx > kPfShiftSlack || (m_run == -INFINITY && mx != -INFINITY);
    if (__ballot(want) != 0) {  // (uniform)
      const float cm = xor_reduce<16, kWave>(mx, [](float x, float y) { return fmaxf(x, y); });
      const bool moved = cm > kPfShiftSlack || (m_run == -INFINITY && cm != -INFINITY);
      const float d = moved ? cm : 0.f;
      const float alpha = m_run == -INFINITY ? 0.f : pf_exp2(-d);
      if (moved) m_run = ref + d;
#pragma unroll
      for (int th = 0; th < 4; ++th)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[th][e] -= d;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
      lacc *= alpha;
    }
    uint32_t pa[4], pb2[4];  // bf16 pairs: keys 16 th + 4 lq + (0, 1) and (2, 3), column lr
#pragma unroll
    for (int th = 0; th < 4; ++th) {
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[e] = pf_exp2(sv[th][e]);
      pa[th] = pack_bf16x2(pv[0], pv[1]);
      pb2[th] = pack_bf16x2(pv[2], pv[3]);
    }
    // The B operand of keys 32 ks .. 32 ks + 31 wants keys 32 ks + 8 lq +
    // (0..7) of column lr in lane (lq, lr): those sit in rows 2 (lq % 2) and
    // 2 (lq % 2) + 1 of slice th = 2 ks + lq / 2.  Swapping rows 2, 3 of
    // slice 2 ks with rows 0, 1 of slice 2 ks + 1, then the odd rows of the
    // first result with the even rows of the second, leaves the first
    // register with rows (0, 2) of each slice and the second with rows
    // (1, 3): the operand's dwords 0 and 2 (dwords 1 and 3 from the (2, 3)
    // pairs).
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const auto a32 = __builtin_amdgcn_permlane32_swap(pa[2 * ks], pa[2 * ks + 1], false, false);
      const auto a16 = __builtin_amdgcn_permlane16_swap(a32[0], a32[1], false, false);
      const auto b32 = __builtin_amdgcn_permlane32_swap(pb2[2 * ks], pb2[2 * ks + 1], false, false);
      const auto b16 = __builtin_amdgcn_permlane16_swap(b32[0], b32[1], false, false);
      pb[ks] = make_uint4(a16[0], b16[0], a16[1], b16[1]);
    }
  };
  // O^T (dims x columns) += V^T (dims x keys) . P (keys x columns), and the
  // column sums from the same P against an all-ones operand
  auto pv_tile = [&](const uint4* pb, PrefillVTile<D>& vc) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] = pf_mfma(vc.u[4 * ks + lq][16 * dt + lr], pb[ks], oacc[dt]);
      lacc = pf_mfma(ones, pb[ks], lacc);
    }
  };

  // Tile `tile`, in buffer B: tile + 1's loads go out into buffer B + 1
  // first (its last reader finished before the barrier that ended the
  // previous tile) and are waited for at the end, before the barrier.
  // Waves 4-7 share SIMDs with waves 0-3 (the dispatcher places waves w and
  // w + 4 of a workgroup on one SIMD) and run the same steps one P.V behind
  // (LAG): they start a tile with the previous tile's P.V, from
  // buffer B - 1, and keep this tile's probabilities for the next.  The two
  // waves of a SIMD are then in different phases (one's MFMAs beside the
  // other's softmax) instead of in step.
  uint4 p_prev[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  auto tile_step = [&](int tile, auto bufc, auto lagc) {
    constexpr int B = decltype(bufc)::value;
    constexpr bool LAG = decltype(lagc)::value;
    PrefillKTile<D>& kc = pf_pick<B>(k0, k1, k2);
    PrefillVTile<D>& vc = pf_pick<B>(v0, v1, v2);
    PrefillKTile<D>& kn = pf_pick<(B + 1) % kPfBufs>(k0, k1, k2);
    PrefillVTile<D>& vn = pf_pick<(B + 1) % kPfBufs>(v0, v1, v2);
    if constexpr (LAG) {
      if (tile > 0) pv_tile(p_prev, pf_pick<(B + kPfBufs - 1) % kPfBufs>(v0, v1, v2));
    }
    const int key0 = tile * kPfTile;
    const bool tile_ok = ok_next;
    st_cur = st_next;
    if (st_cur != rot_st) {  // Rot(n - st) q = Rot(-st) Rot(n) q, split into bf16 hi + lo
      rot_st = st_cur;
      float hi[NCH][8], lo[NCH][8];
#pragma unroll
      for (int c = 0; c < NCH / 2; ++c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 32 * c + 8 * lq + e;
          const float cv = sh.cs[B][d][0], sv = sh.cs[B][d][1];
          const float x1 = qn[c][e], x2 = qn[c + NCH / 2][e];
          const float r1 = x1 * cv + x2 * sv, r2 = x2 * cv - x1 * sv;
          hi[c][e] = round_bf16(r1);
          hi[c + NCH / 2][e] = round_bf16(r2);
          lo[c][e] = r1 - hi[c][e];
          lo[c + NCH / 2][e] = r2 - hi[c + NCH / 2][e];
        }
      }
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        qhi[c] = pack_bf16x8(hi[c]);
        qlo[c] = pack_bf16x8(lo[c]);
      }
    }
    if (tile + 1 < ntile) {
      tile_page(tile + 1, page, st);
      fetch_lds(tile + 1, page, kn, vn);
    }

    // A tile inside the context and at or before every column's position
    // (all but the last few) needs no mask.
    const bool full = tile_ok && key0 + kPfTile <= T && (int64_t)(key0 + kPfTile - 1) <= p0 + m0;
    pf_floatx4 acc[4];
    qk_tile(kc, acc);
    uint4 pb[2];
    softmax_tile(acc, key0, tile_ok, full, pb);
    if constexpr (LAG) {
      p_prev[0] = pb[0];
      p_prev[1] = pb[1];
    } else {
      pv_tile(pb, vc);
    }

    // tile + 1 complete in the next buffer, with its rotation table where
    // its document differs from tile's (read only there, as every wave's
    // rotation); the next run of tile pages before its first lookup
    if (tile + 1 < ntile) {
      ok_next = page >= 0;
      st_next = st;
      if (st_next != st_cur) rotation_table(st_next, (B + 1) % kPfBufs);
      wait_loads();
      mask_tail(tile + 1, vn);
      if ((tile + 2) % kPfThreads == 0 && tile + 2 < ntile) {  // (uniform)
        __syncthreads();  // every lookup in the current run done
        resolve_run((tile + 2) / kPfThreads);
      }
    }
    __syncthreads();  // tile + 1 and its table complete; buffer B - 1 free
  };
  // the buffers rotate with period three, so each step names its buffers
  // statically
  auto run_tiles = [&](auto lagc) {
    for (int tile = 0; tile < ntile; tile += kPfBufs) {
      tile_step(tile, PfBuf<0>{}, lagc);
      if (tile + 1 < ntile) tile_step(tile + 1, PfBuf<1>{}, lagc);
      if (tile + 2 < ntile) tile_step(tile + 2, PfBuf<2>{}, lagc);
    }
  };
  if (wu >= kPfWaves / 2) {
    run_tiles(std::true_type{});
    if (ntile > 0) {  // the last tile's P.V
      const int lb = (ntile - 1) % kPfBufs;
      if (lb == 0)
        pv_tile(p_prev, v0);
      else if (lb == 1)
        pv_tile(p_prev, v1);
      else
        pv_tile(p_prev, v2);
    }
  } else {
    run_tiles(std::false_type{});
  }

  // column totals
  const float lsum = lacc[0];
  m_hi = xor_reduce<16, kWave>(m_hi, [](float x, float y) { return fmaxf(x, y); });  // the column's
  if (col_ok) {
    const int64_t row = ((int64_t)b * a.M + mi) * a.Hq + (int64_t)h * G + g;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.o[row * D + 16 * dt + 4 * lq + e] = oacc[dt][e] * inv;
    if (lq == 0) {
      // the sum against the exact max: m_run trails m_hi by at most the slack
      a.m[row] = lsum > 0.f ? m_hi * kPfLn2 : -INFINITY;
      a.l[row] = lsum > 0.f ? lsum * exp2f(m_run - m_hi) : lsum;
    }
  }
}

template <int D>
static void launch_prefill_d(dim3 grid, const PrefillArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: prefill_rope_kernel<D, 1><<<grid, kPfThreads, 0, stream>>>(a); break;
    case 2: prefill_rope_kernel<D, 2><<<grid, kPfThreads, 0, stream>>>(a); break;
    case 4: prefill_rope_kernel<D, 4><<<grid, kPfThreads, 0, stream>>>(a); break;
    case 8: prefill_rope_kernel<D, 8><<<grid, kPfThreads, 0, stream>>>(a); break;
    default: prefill_rope_kernel<D, 16><<<grid, kPfThreads, 0, stream>>>(a); break;
  }
}

hipError_t launch_prefill_attention(const nosa_dims& d, const nosa_kv& kv, const uint16_t* q, int32_t n_prompt,
                                    const int32_t* q_pos0, const int32_t* seq_lens, float sm_scale, float* o,
                                    float* m, float* l, hipStream_t stream) {
  PrefillArgs a;
  a.t = make_table(d, kv);
  a.Hq = d.n_q_heads;
  a.bs = d.block_size;
  a.M = n_prompt;
  a.scale_log2 = sm_scale * kPfLog2e;
  a.rope_base = (double)kv.rope_base;
  a.q = q;
  a.k_pages = kv.k_pages;
  a.v_pages = kv.v_pages;
  a.q_pos0 = q_pos0;
  a.seq_lens = seq_lens;
  a.o = o;
  a.m = m;
  a.l = l;
  const int G = d.n_q_heads / d.n_kv_heads;
  const int rows_per_wg = kPfWaves * (kPfCols / G);
  a.n_chunks = (n_prompt + rows_per_wg - 1) / rows_per_wg;
  a.n_pairs = d.batch * d.n_kv_heads;
  const int64_t total = (int64_t)a.n_chunks * a.n_pairs;
  const dim3 grid((unsigned)((total + kPfXcds - 1) / kPfXcds * kPfXcds));
  if (d.head_dim == 128)
    launch_prefill_d<128>(grid, a, G, stream);
  else
    launch_prefill_d<64>(grid, a, G, stream);
  return hipGetLastError();
}

}  // namespace nosa
