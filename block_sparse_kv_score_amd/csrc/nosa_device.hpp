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

// Data that other workgroups of the same launch read back.  Device-scope
// (agent) atomic stores are made visible across every XCD's L2 before they
// complete, and device-scope atomic loads never hit a stale L2 line, so a
// producer needs only to wait for its stores to complete (s_waitcnt
// vmcnt(0)) before it signals, and no L2 write-back or invalidate is
// needed on either side.
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

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, kWave));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace nosa
