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
// through a double-buffered LDS tile (eight waves rather than four halve the
// tile loads and stores per column; the register file holds two waves per
// SIMD, so one workgroup per CU): tile t + 1, loaded into registers while
// tile t - 1 was used, is stored into the other buffer after tile t's
// products, one workgroup barrier per tile.  Workgroups are placed
// XCD-aware: the workgroups of one (b, KV head) run on one XCD, so its K and
// V stream from that XCD's L2 after the first reader.  Both products run on v_mfma_f32_16x16x32_bf16 as in the
// decode: S^T = K . Q^T with the key rows as the A operand straight from the
// K page layout, and O^T += V^T . P with V^T rows from the V page layout and
// the tile's bf16 probabilities (one LDS round trip) as the B operand.  The
// rotated query is split into bf16 hi + lo parts (two MFMAs per chunk) so the
// rotation costs no precision beyond ~2^-16.  Online softmax per column in
// log2 units; causal mask t <= n; keys past the context are masked and their
// V entries zeroed (0 * stale NaN would leak through the MFMA).

#include "nosa_device.hpp"
#include "nosa_launch.hpp"

namespace nosa {

constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfTile = 64;  // keys per tile
constexpr int kPfCols = 16;  // query columns per wave
// Row pitch of the per-wave probability tile, in bf16: 64 keys + 8 of
// padding, so the 16 lanes of a row group (one column each) fall on
// distinct LDS banks (a 128-byte pitch would put every other column on the
// same banks).
constexpr int kPfPitch = kPfTile + 8;
constexpr int kPfXcds = 8;  // XCDs: consecutive workgroups go to consecutive XCDs
constexpr float kPfLog2e = 1.4426950408889634f;
constexpr float kPfLn2 = 0.6931471805599453f;

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
struct PrefillSmem {
  uint4 k[2][D / 8][kPfTile];                  // K tiles, page layout [D/8][64][8]
  uint4 v[2][kPfTile / 8][D];                  // V tiles, page layout [64/8][D][8]
  uint16_t p[kPfWaves][kPfCols][kPfPitch];     // bf16 probabilities, per wave
  float cs[2][D / 2][2];                       // cos, sin of st * theta_k, per buffer
};

typedef __bf16 pf_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pf_floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ pf_floatx4 pf_mfma(const uint4& a, const uint4& b, const pf_floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pf_bf16x8, a), __builtin_bit_cast(pf_bf16x8, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ uint4 pf_load(const uint4* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
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
  __shared__ PrefillSmem<D> sh;

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
  float m_run = -INFINITY, l_run = 0.f;  // column lr, log2 units (l_run: this lane's keys)
  pf_floatx4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = pf_floatx4{0.f, 0.f, 0.f, 0.f};

  // tile -> page and document start (tokens); page < 0: unresolvable
  auto tile_page = [&](int tile, int64_t& page, int64_t& st) {
    const int i = tile * kPfTile / bs;
    uint32_t docb = 0;
    page = page_of<NOSA_TABLE_PACKED_ROPE>(t, bh, i, docb);
    st = (int64_t)docb * bs;
  };
  uint4 kr[KU], vr[VU];
  auto fetch = [&](int tile, int64_t page) {
    const int sub = (tile * kPfTile % bs) / kPfTile;
    const uint4* kp = reinterpret_cast<const uint4*>(a.k_pages + page * (int64_t)bs * D);
    const uint4* vp = reinterpret_cast<const uint4*>(a.v_pages + page * (int64_t)bs * D);
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int u = threadIdx.x + j * kPfThreads;
      kr[j] = page >= 0 ? pf_load(kp + (int64_t)(u / kPfTile) * bs + sub * kPfTile + u % kPfTile)
                        : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = threadIdx.x + j * kPfThreads;
      vr[j] = page >= 0 ? pf_load(vp + (int64_t)(sub * 8 + u / D) * D + u % D) : make_uint4(0, 0, 0, 0);
    }
  };

  // the registers of tile `tile` into LDS buffer `buf` (V past the context zeroed)
  auto stage = [&](int tile, int buf) {
    const int key0 = tile * kPfTile;
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int u = threadIdx.x + j * kPfThreads;
      sh.k[buf][u / kPfTile][u % kPfTile] = kr[j];
    }
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = threadIdx.x + j * kPfThreads;
      const int ko = u / D;
      uint4 x = vr[j];
      const int nv = min(max(T - (key0 + 8 * ko), 0), 8);  // present keys of this unit
      if (nv < 8) {
        uint32_t mk[4];
#pragma unroll
        for (int jd = 0; jd < 4; ++jd)
          mk[jd] = (2 * jd < nv ? 0x0000ffffu : 0u) | (2 * jd + 1 < nv ? 0xffff0000u : 0u);
        x.x &= mk[0];
        x.y &= mk[1];
        x.z &= mk[2];
        x.w &= mk[3];
      }
      sh.v[buf][ko][u % D] = x;
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

  // prologue: tile 0 in buffer 0 with its rotation table, tile 1 in flight
  int64_t page = -1, st = 0;         // the tile in the registers
  int64_t st_cur = -1, st_next = 0;  // document starts of tiles t and t + 1
  bool ok_next = false;              // tile t + 1 resolvable
  if (ntile > 0) {
    tile_page(0, page, st);
    if (page < 0 && threadIdx.x == 0) flag_error(t.err);
    fetch(0, page);
    stage(0, 0);
    rotation_table(st, 0);
    st_next = st;
    ok_next = page >= 0;
    if (ntile > 1) {
      tile_page(1, page, st);
      if (page < 0 && threadIdx.x == 0) flag_error(t.err);
      fetch(1, page);
    }
  }
  __syncthreads();

  int64_t rot_st = -1;  // the document start qhi / qlo are rotated for
  for (int tile = 0; tile < ntile; ++tile) {
    const int buf = tile & 1;
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
          const float cv = sh.cs[buf][d][0], sv = sh.cs[buf][d][1];
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

    // S^T: rows = keys 16 th + 4 lq + e of the tile, column lr.  A tile
    // inside the context and at or before every column's position (all but
    // the last few) needs no mask.
    const bool full = tile_ok && key0 + kPfTile <= T && (int64_t)(key0 + kPfTile - 1) <= p0 + m0;
    // chunk-major order: the four key slices' accumulators are independent,
    // so consecutive MFMAs do not wait on each other's results
    pf_floatx4 acc[4];
#pragma unroll
    for (int th = 0; th < 4; ++th) acc[th] = pf_floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      uint4 ka[4];
#pragma unroll
      for (int th = 0; th < 4; ++th) ka[th] = sh.k[buf][4 * c + lq][16 * th + lr];
#pragma unroll
      for (int th = 0; th < 4; ++th) acc[th] = pf_mfma(ka[th], qhi[c], acc[th]);
#pragma unroll
      for (int th = 0; th < 4; ++th) acc[th] = pf_mfma(ka[th], qlo[c], acc[th]);
    }
    float sv[4][4];
#pragma unroll
    for (int th = 0; th < 4; ++th)
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[th][e] = acc[th][e];
    if (!full) {  // (uniform) key 16 th + 4 lq + e is visible iff 16 th + e <= lim
      const int64_t lim64 = min((int64_t)T - 1, n) - (key0 + 4 * lq);
      const int lim = tile_ok ? (int)max(min(lim64, (int64_t)kPfTile), (int64_t)-1) : -1;
#pragma unroll
      for (int th = 0; th < 4; ++th)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[th][e] = 16 * th + e <= lim ? sv[th][e] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int th = 0; th < 4; ++th)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sv[th][e]);
    mx = xor_reduce<16, kWave>(mx, [](float x, float y) { return fmaxf(x, y); });
    const float mn = fmaxf(m_run, mx);
    // a column with every key so far masked has mn = -inf: exponents are then
    // taken against 0 (masked scores are -inf, so they still give 0 and no
    // NaN arises; alpha = 0 scales an all-zero accumulator)
    const float mz = mn == -INFINITY ? 0.f : mn;
    const float alpha = pf_exp2(m_run - mz);
    m_run = mn;
    float psum = 0.f;
#pragma unroll
    for (int th = 0; th < 4; ++th) {
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv[e] = pf_exp2(sv[th][e] - mz);
        psum += pv[e];
      }
      const uint32_t w0 = pack_bf16x2(pv[0], pv[1]);
      const uint32_t w1 = pack_bf16x2(pv[2], pv[3]);
      *reinterpret_cast<uint2*>(&sh.p[w][lr][16 * th + 4 * lq]) = make_uint2(w0, w1);
    }
    l_run = l_run * alpha + psum;
    if (__ballot(alpha != 1.f) != 0) {  // (a product with 1 changes nothing)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
    }
    wave_lds_sync();

    // O^T (dims x columns) += V^T (dims x keys) . P (keys x columns)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 pb = *reinterpret_cast<const uint4*>(&sh.p[w][lr][32 * ks + 8 * lq]);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] = pf_mfma(sh.v[buf][4 * ks + lq][16 * dt + lr], pb, oacc[dt]);
    }

    // tile + 1 (in the registers) into the other buffer, with its rotation
    // table where its document differs from tile's (read only there, as
    // every wave's rotation); tile + 2's loads go out
    if (tile + 1 < ntile) {
      ok_next = page >= 0;
      stage(tile + 1, buf ^ 1);
      st_next = st;
      if (st_next != st_cur) rotation_table(st_next, buf ^ 1);
      if (tile + 2 < ntile) {
        tile_page(tile + 2, page, st);
        if (page < 0 && threadIdx.x == 0) flag_error(t.err);
        fetch(tile + 2, page);
      }
    }
    __syncthreads();  // buffer buf ^ 1 and its table complete; buffer buf free
  }

  // column totals: l over the lanes that share the column
  const float lsum = xor_reduce<16, kWave>(l_run, [](float x, float y) { return x + y; });
  if (col_ok) {
    const int64_t row = ((int64_t)b * a.M + mi) * a.Hq + (int64_t)h * G + g;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.o[row * D + 16 * dt + 4 * lq + e] = oacc[dt][e] * inv;
    if (lq == 0) {
      a.m[row] = lsum > 0.f ? m_run * kPfLn2 : -INFINITY;
      a.l[row] = lsum;
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
