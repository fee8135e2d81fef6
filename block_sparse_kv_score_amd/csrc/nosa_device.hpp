// Device-side helpers shared by the libnosa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nosa.h"

namespace nosa {

constexpr int kWave = 64;

// Logical block -> physical page, for every table kind.  Passed by value.
struct Table {
  int32_t kind;
  int32_t Hkv;
  int32_t max_blocks;
  int32_t dir_entries;
  int32_t seg_log2;
  int32_t blocks_log2;
  int64_t num_pages;
  int64_t num_segments;
  const int32_t* table;
  const int32_t* directory;
  const int32_t* segments;
  const uint32_t* packed;
  int32_t* err;
};

// The table descriptor of a call (defined with the index kernels).
Table make_table(const nosa_dims& d, const nosa_kv& kv);

__device__ __forceinline__ void flag_error(int32_t* err) {
  if (err) atomicOr(err, 1);
}

// Page of logical block i of pair bh, or -1 when the table holds no valid
// page for it.  For the packed kind, doc_blocks receives the document start
// (in blocks) stored beside the page id.
template <int KIND>
__device__ __forceinline__ int64_t page_of(const Table& t, int bh, int i, uint32_t& doc_blocks) {
  int64_t page;
  if constexpr (KIND == NOSA_TABLE_FLAT) {
    page = t.table[(int64_t)bh * t.max_blocks + i];
  } else if constexpr (KIND == NOSA_TABLE_TWO_LEVEL) {
    const int64_t key = ((int64_t)bh << t.blocks_log2) | (int64_t)i;
    const int64_t d = key >> t.seg_log2;
    if (d >= t.dir_entries) return -1;
    const int32_t seg = t.directory[d];
    if (seg < 0 || seg >= t.num_segments) return -1;
    page = t.segments[((int64_t)seg << t.seg_log2) | (key & ((1ll << t.seg_log2) - 1))];
  } else {
    const uint32_t w = t.packed[(int64_t)bh * t.max_blocks + i];
    page = (int64_t)(w & ((1u << NOSA_PACK_PAGE_BITS) - 1u));
    doc_blocks = w >> NOSA_PACK_PAGE_BITS;
  }
  if (page < 0 || page >= t.num_pages) return -1;
  return page;
}

__device__ __forceinline__ int64_t page_of_any(const Table& t, int bh, int i, uint32_t& doc_blocks) {
  switch (t.kind) {
    case NOSA_TABLE_FLAT: return page_of<NOSA_TABLE_FLAT>(t, bh, i, doc_blocks);
    case NOSA_TABLE_TWO_LEVEL: return page_of<NOSA_TABLE_TWO_LEVEL>(t, bh, i, doc_blocks);
    default: return page_of<NOSA_TABLE_PACKED_ROPE>(t, bh, i, doc_blocks);
  }
}

// bf16 halves of a 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Orders fp32 scores as unsigned integers: a > b  <=>  key(a) > key(b).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of set bits of a wave ballot below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Orders LDS traffic between lanes of one wave (LDS executes a wave's
// operations in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Data that other workgroups of the same launch read back (the split
// partials of the fused combine, the tile statistics of the softmax score
// step).  The rule this relies on, in ISA terms: the compiler's AMDGPU
// memory model for the gfx942 family (gfx950 included) lowers a relaxed
// agent-scope atomic store or load to a single global_store / global_load
// with the sc1 (agent-scope coherence) bit set and no cache maintenance
// around it -- the sc1 bit alone makes that location's accesses coherent
// across the device's L1s and the L2s of all XCDs.  The decode's code is
// `global_store_dword ... sc1` for the partials, `global_atomic_add ...
// sc0` (old value returned) for the arrival counter and `global_load_dword
// ... sc1` for the read-back.  The protocol: every wave of a producer waits
// for vmcnt(0), i.e. until its sc1 stores have completed, then the
// workgroup barrier, then one thread adds to the counter; the workgroup
// that gets P - 1 back issues its sc1 loads only after that atomic has
// returned (its value decides the branch).  A completed sc1 store is seen
// by every later sc1 load of the same location anywhere on the device, so
// the last workgroup reads every partial.  The C++ orderings are relaxed
// on purpose: the wait orders the accesses; a release / acquire pair would
// add an L2 write-back (buffer_wbl2 sc1) and invalidate (buffer_inv sc1)
// that data written and read only through sc1 accesses does not need.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Plain load, or a device-scope atomic load of data written by other
// workgroups of the same launch with store_coherent.
template <bool COHERENT>
__device__ __forceinline__ float load_f32(const float* p) {
  if constexpr (COHERENT)
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

// s_waitcnt immediate (gfx9 family encoding) that waits for every vector
// memory operation of the wave, stores included, and leaves the other
// counters unconstrained: vmcnt = 0, expcnt = 7, lgkmcnt = 15.
constexpr int kWaitVmcnt0 = (0xF << 8) | (0x7 << 4);

// ---------------------------------------------------------------------------
// Cross-lane exchanges in registers.  HIP's __shfl family goes through the
// LDS crossbar (ds_bpermute), one dependent LDS round trip per step; these
// use DPP row operations and the gfx950 permlane swaps instead (lane
// layouts as documented for CDNA: quad_perm, row_shl/shr/ror within rows of
// 16 lanes, row_bcast:15/31 across rows, v_permlane16/32_swap exchanging
// rows / halves between two registers).
// ---------------------------------------------------------------------------

// The value of lane (this lane ^ M), M a power of two below 64.
template <int M>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v) {
  const int x = (int)v;
  if constexpr (M == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    const int up = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xf, 0xf, false);  // row_shl:4: lane i <- i + 4
    const int dn = __builtin_amdgcn_update_dpp(x, x, 0x114, 0xf, 0xf, false);  // row_shr:4: lane i <- i - 4
    return (uint32_t)((threadIdx.x & 4) ? dn : up);
  } else if constexpr (M == 8) {
    return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x128, 0xf, 0xf, false);  // row_ror:8
  } else if constexpr (M == 16) {
    // with both operands x: [0] = rows (0,0,2,2), [1] = rows (1,1,3,3)
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (uint32_t)((threadIdx.x & 16) ? p[0] : p[1]);
  } else {
    static_assert(M == 32, "lane_xor: M in {1, 2, 4, 8, 16, 32}");
    // with both operands x: [0] = halves (0,0), [1] = halves (1,1)
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (uint32_t)((threadIdx.x & 32) ? p[0] : p[1]);
  }
}

template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  return __uint_as_float(lane_xor_u32<M>(__float_as_uint(v)));
}
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  return lane_xor_u32<M>(v);
}
template <int M>
__device__ __forceinline__ double lane_xor(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint64_t lo = lane_xor_u32<M>((uint32_t)u), hi = lane_xor_u32<M>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(lo | (hi << 32)));
}

// v = op(v, v of lane ^ M) for M = FROM, 2 FROM, .. < TO: the reduction over
// the lanes that agree with this one outside bits [log2 FROM, log2 TO), in
// the same order as the classic butterfly.
template <int FROM, int TO, typename T, typename Op>
__device__ __forceinline__ T xor_reduce(T v, Op op) {
  if constexpr (FROM < TO) {
    v = op(v, lane_xor<FROM>(v));
    return xor_reduce<FROM * 2, TO>(v, op);
  } else {
    return v;
  }
}

// As xor_reduce<1, 64>, but only over bits below log2 n (n a power of two,
// 1 <= n <= 64, uniform at run time).
template <typename T, typename Op>
__device__ __forceinline__ T xor_reduce_below(T v, int n, Op op) {
  if (n > 1) v = op(v, lane_xor<1>(v));
  if (n > 2) v = op(v, lane_xor<2>(v));
  if (n > 4) v = op(v, lane_xor<4>(v));
  if (n > 8) v = op(v, lane_xor<8>(v));
  if (n > 16) v = op(v, lane_xor<16>(v));
  if (n > 32) v = op(v, lane_xor<32>(v));
  return v;
}

// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ int wave_scan_incl(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1 (row start reads 0)
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2 and 3
  return x;
}

}  // namespace nosa
