// Retrieve: the host tier of the paged KV cache.
//
// NOSA summary (gist.science 2510.13602), Methodology 2 (NOSI): the KV cache
// is kept in block-sized units, set differences between consecutive block
// sets drive block swapping, and a custom host-to-device transfer kernel
// over unified virtual addressing reaches near-peak PCIe bandwidth.  Spin
// summary (gist.science 2604.26837), 2.A: Offload (place data in memory)
// and Retrieve (fetch it from CPU memory) are system-managed operations on
// the shared page substrate; 2.B: pages are per head, so only relevant data
// crosses the host link.
//
// Layout.  The whole paged cache (K, V, E pages, same layouts as the device
// pools) lives in pinned host memory, addressed by the logical table of a
// nosa_kv descriptor.  HBM holds a resident pool of RS pages per (b, h):
// device page bh * RS + s is slot s of pair bh.  The resident table maps a
// logical block to its device page (or -1) and slot_owner maps a slot back
// to its block (or -1); together they are the pair's resident set.
//
// One workgroup per (b, h):
//   1. every evicted block gives its slot back;
//   2. the free slots are numbered in ascending order and the j-th loaded
//      block takes the j-th free one (a deterministic assignment);
//   3. the loaded blocks' K, V and E pages are read straight from host
//      memory (zero-copy, 16 bytes per lane, several loads in flight per
//      thread) into their slots; the resident tail block (the one the
//      append wrote into, in host memory) is copied again so its new token
//      reaches HBM.

#include "nosa_launch.hpp"

namespace nosa {

constexpr int kRetrieveThreads = 256;
constexpr int kRetrieveBatch = 8;  // 16-byte copies in flight per thread

struct RetrieveArgs {
  Table host;  // logical block -> page of the host pools
  const uint4* hk;
  const uint4* hv;
  const uint4* he;
  uint4* dk;
  uint4* dv;
  uint4* de;
  int RS, bs, D, cap;
  int32_t* resident;  // [B][Hkv][max_blocks]
  int32_t* owner;     // [B][Hkv][RS]
  const int32_t* load;
  const int32_t* load_count;
  const int32_t* evict;
  const int32_t* evict_count;
  const int32_t* seq_lens;
};

__global__ __launch_bounds__(kRetrieveThreads) void retrieve_kernel(const RetrieveArgs a) {
  __shared__ int32_t free_slot[kMaxRetrieveSlots];
  __shared__ int64_t src_page[kMaxRetrieveSlots + 1];
  __shared__ int32_t dst_page[kMaxRetrieveSlots + 1];
  __shared__ int32_t wave_tot[kRetrieveThreads / kWave];
  __shared__ int32_t n_copy;
  const Table& t = a.host;
  const int bh = blockIdx.x;
  const int b = bh / t.Hkv;
  const int MB = t.max_blocks, RS = a.RS;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int32_t* res = a.resident + (int64_t)bh * MB;
  int32_t* own = a.owner + (int64_t)bh * RS;
  const int page0 = bh * RS;

  // 1. evictions give their slots back
  const int ne = min(max(a.evict_count[bh], 0), a.cap);
  for (int k = threadIdx.x; k < ne; k += kRetrieveThreads) {
    const int x = a.evict[(int64_t)bh * a.cap + k];
    if (x < 0 || x >= MB) continue;
    const int p = res[x];
    if (p >= page0 && p < page0 + RS) own[p - page0] = -1;
    res[x] = -1;
  }
  __syncthreads();

  // 2. free slots in ascending order: thread t scans slots [4t, 4t + 4)
  //    (RS <= 4 * 256), then a workgroup prefix sum places them
  int fr[4], nf = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = 4 * threadIdx.x + j;
    fr[j] = s < RS && own[s] < 0;
    nf += fr[j];
  }
  const int incl = wave_scan_incl(nf);
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int base = incl - nf;
#pragma unroll
  for (int ww = 0; ww < kRetrieveThreads / kWave; ++ww) base += ww < w ? wave_tot[ww] : 0;
  int n_free = 0;
#pragma unroll
  for (int ww = 0; ww < kRetrieveThreads / kWave; ++ww) n_free += wave_tot[ww];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (fr[j]) free_slot[base++] = 4 * threadIdx.x + j;
  }
  __syncthreads();

  // 3. loaded blocks take the free slots in order
  int nl = min(max(a.load_count[bh], 0), a.cap);
  if (nl > n_free) {
    if (threadIdx.x == 0) flag_error(t.err);
    nl = n_free;
  }
  for (int j = threadIdx.x; j < nl; j += kRetrieveThreads) {
    const int y = a.load[(int64_t)bh * a.cap + j];
    int64_t hp = -1;
    int dp = -1;
    if (y >= 0 && y < MB) {
      uint32_t doc;
      hp = page_of_any(t, bh, y, doc);
      const int s = free_slot[j];
      own[s] = y;
      res[y] = page0 + s;
      dp = page0 + s;
    }
    if (hp < 0) flag_error(t.err);
    src_page[j] = hp < 0 ? -1 : hp;
    dst_page[j] = hp < 0 ? -1 : dp;
  }
  __syncthreads();
  // the resident tail block: the append wrote its new token into host memory
  if (threadIdx.x == 0) {
    int nc = nl;
    const int T = min(max(a.seq_lens[b], 0), MB * a.bs);
    if (T > 0) {
      const int tb = (T - 1) / a.bs;
      const int p = res[tb];
      if (p >= page0 && p < page0 + RS) {
        uint32_t doc;
        const int64_t hp = page_of_any(t, bh, tb, doc);
        if (hp >= 0) {
          src_page[nc] = hp;
          dst_page[nc] = p;
          ++nc;
        } else {
          flag_error(t.err);
        }
      }
    }
    n_copy = nc;
  }
  __syncthreads();

  // 4. copy: K, V and E of each page as 16-byte units
  const int ku = a.bs * a.D / 8;  // units of a K (or V) page
  const int eu = a.bs / 4;        // units of an E page
  const int upb = 2 * ku + eu;
  const int total = n_copy * upb;
  for (int u0 = threadIdx.x; u0 < total; u0 += kRetrieveThreads * kRetrieveBatch) {
    uint4 v[kRetrieveBatch];
    const uint4* src[kRetrieveBatch];
    uint4* dst[kRetrieveBatch];
#pragma unroll
    for (int k = 0; k < kRetrieveBatch; ++k) {
      const int u = min(u0 + k * kRetrieveThreads, total - 1);  // clamped: loads need no branch
      const int j = u / upb, r = u % upb;
      const int64_t hp = src_page[j];
      const int64_t dp = dst_page[j];
      if (r < ku) {
        src[k] = a.hk + hp * ku + r;
        dst[k] = a.dk + dp * ku + r;
      } else if (r < 2 * ku) {
        src[k] = a.hv + hp * ku + (r - ku);
        dst[k] = a.dv + dp * ku + (r - ku);
      } else {
        src[k] = a.he + hp * eu + (r - 2 * ku);
        dst[k] = a.de + dp * eu + (r - 2 * ku);
      }
      v[k] = hp >= 0 ? *src[k] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kRetrieveBatch; ++k) {
      const int u = u0 + k * kRetrieveThreads;
      if (u < total && src_page[u / upb] >= 0) *dst[k] = v[k];
    }
  }
}

hipError_t launch_retrieve(const nosa_dims& d, const nosa_kv& host_kv, const void* host_k, const void* host_v,
                           const void* host_e, uint16_t* dev_k, uint16_t* dev_v, float* dev_e, int32_t slots,
                           int32_t* resident, int32_t* slot_owner, const int32_t* load, const int32_t* load_count,
                           const int32_t* evict, const int32_t* evict_count, int32_t cap, const int32_t* seq_lens,
                           hipStream_t stream) {
  RetrieveArgs a;
  a.host = make_table(d, host_kv);
  a.hk = reinterpret_cast<const uint4*>(host_k);
  a.hv = reinterpret_cast<const uint4*>(host_v);
  a.he = reinterpret_cast<const uint4*>(host_e);
  a.dk = reinterpret_cast<uint4*>(dev_k);
  a.dv = reinterpret_cast<uint4*>(dev_v);
  a.de = reinterpret_cast<uint4*>(dev_e);
  a.RS = slots;
  a.bs = d.block_size;
  a.D = d.head_dim;
  a.cap = cap;
  a.resident = resident;
  a.owner = slot_owner;
  a.load = load;
  a.load_count = load_count;
  a.evict = evict;
  a.evict_count = evict_count;
  a.seq_lens = seq_lens;
  retrieve_kernel<<<d.batch * d.n_kv_heads, kRetrieveThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace nosa
