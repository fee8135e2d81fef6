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
//      thread) into their slots; resident blocks that took appended tokens
//      in host memory since the previous retrieve get those tokens copied
//      (or, without the previous lengths, the tail block whole).

#include "nosa_device.hpp"
#include "nosa_launch.hpp"

namespace nosa {

constexpr int kRetrieveThreads = 256;
constexpr int kRetrieveBatch = 8;  // 16-byte copies in flight per thread
constexpr int kRecencyBuckets = 64;

// Copies n pages (K, V and E of each) from the host pools to the resident
// pools as 16-byte units, kRetrieveBatch loads in flight per thread.
// src_page[j] < 0 skips page j.  ku: units of a K (or V) page; eu: of an E
// page.
__device__ __forceinline__ void copy_pages(const uint4* hk, const uint4* hv, const uint4* he, uint4* dk, uint4* dv,
                                           uint4* de, int ku, int eu, int n, const int64_t* src_page,
                                           const int32_t* dst_page) {
  const int upb = 2 * ku + eu;
  const int total = n * upb;
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
        src[k] = hk + hp * ku + r;
        dst[k] = dk + dp * ku + r;
      } else if (r < 2 * ku) {
        src[k] = hv + hp * ku + (r - ku);
        dst[k] = dv + dp * ku + (r - ku);
      } else {
        src[k] = he + hp * eu + (r - 2 * ku);
        dst[k] = de + dp * eu + (r - 2 * ku);
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

// Workgroup-wide exclusive prefix sum of one count per thread (every thread
// calls it; wave_tot holds a wave's total).  Returns this thread's offset;
// *total receives the sum.
__device__ __forceinline__ int workgroup_offset(int x, int32_t* wave_tot, int* total) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int incl = wave_scan_incl(x);
  __syncthreads();  // wave_tot may still be read from a previous call
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int base = incl - x, sum = 0;
#pragma unroll
  for (int ww = 0; ww < kRetrieveThreads / kWave; ++ww) {
    base += ww < w ? wave_tot[ww] : 0;
    sum += wave_tot[ww];
  }
  *total = sum;
  return base;
}

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
  const int32_t* seq_prev;  // [B] or null
};

// Plans the refresh of resident pages whose host copy took appended tokens
// since the previous retrieve (the append writes into the host pools).
// lo >= 0: the tokens [lo, T) are new; every resident block holding some of
// them, unless loaded whole by this call, gets those tokens copied.  lo < 0:
// the resident tail block is copied whole.  Entries go to src_page /
// dst_page / rng from index `first` on (rng = first token | end << 16);
// *n_ref (LDS, zero on entry) counts them.  Every thread calls it.
__device__ __forceinline__ void plan_refresh(const Table& t, int bh, int T, int lo, int bs, const int32_t* res,
                                             const uint8_t* fresh, int page0, int RS, int first, int64_t* src_page,
                                             int32_t* dst_page, int32_t* rng, int32_t* n_ref) {
  if (T <= 0) return;
  const int x0 = lo >= 0 ? min(lo, T) / bs : (T - 1) / bs;
  const int x1 = lo >= 0 && lo >= T ? x0 - 1 : (T - 1) / bs;
  for (int x = x0 + (int)threadIdx.x; x <= x1; x += kRetrieveThreads) {
    const int p = res[x];
    if (p < page0 || p >= page0 + RS || fresh[p - page0]) continue;
    uint32_t doc;
    const int64_t hp = page_of_any(t, bh, x, doc);
    if (hp < 0) {
      flag_error(t.err);
      continue;
    }
    const int i = first + atomicAdd(n_ref, 1);
    const int a = lo >= 0 ? max(lo, x * bs) - x * bs : 0;
    const int e = lo >= 0 ? min(T, (x + 1) * bs) - x * bs : bs;
    src_page[i] = hp;
    dst_page[i] = p;
    rng[i] = a | (e << 16);
  }
}

// Copies the tokens [a, e) of each planned page: for K ([D/8][bs][8]) the
// D/8 units of each token, for V ([bs/8][D][8]) the rows of 8 tokens that
// hold them, for E ([bs] fp32) the 4-token units that hold them.
__device__ __forceinline__ void refresh_tokens(const uint4* hk, const uint4* hv, const uint4* he, uint4* dk,
                                               uint4* dv, uint4* de, int bs, int D, int first, int n,
                                               const int64_t* src_page, const int32_t* dst_page,
                                               const int32_t* rng) {
  const int ku = bs * D / 8, eu = bs / 4;
  for (int r = first; r < first + n; ++r) {
    const int64_t hp = src_page[r], dp = dst_page[r];
    const int a = rng[r] & 0xffff, e = rng[r] >> 16;
    const int w = e - a;
    const int nk = (D / 8) * w;
    const int v0 = (a / 8) * D, nv = ((e - 1) / 8 + 1) * D - v0;
    const int e0 = a / 4, ne = (e - 1) / 4 + 1 - e0;
    for (int u = threadIdx.x; u < nk + nv + ne; u += kRetrieveThreads) {
      if (u < nk) {
        const int off = (u / w) * bs + a + u % w;
        dk[dp * ku + off] = hk[hp * ku + off];
      } else if (u < nk + nv) {
        const int off = v0 + (u - nk);
        dv[dp * ku + off] = hv[hp * ku + off];
      } else {
        const int off = e0 + (u - nk - nv);
        de[dp * eu + off] = he[hp * eu + off];
      }
    }
  }
}

__global__ __launch_bounds__(kRetrieveThreads) void retrieve_kernel(const RetrieveArgs a) {
  __shared__ int32_t free_slot[kMaxRetrieveSlots];
  __shared__ int64_t src_page[kMaxRetrieveSlots + 1];
  __shared__ int32_t dst_page[kMaxRetrieveSlots + 1];
  __shared__ int32_t wave_tot[kRetrieveThreads / kWave];
  __shared__ int32_t rng[kMaxRetrieveSlots + 1];
  __shared__ uint8_t fresh[kMaxRetrieveSlots];
  __shared__ int32_t n_ref;
  const Table& t = a.host;
  const int bh = blockIdx.x;
  const int b = bh / t.Hkv;
  const int MB = t.max_blocks, RS = a.RS;
  int32_t* res = a.resident + (int64_t)bh * MB;
  int32_t* own = a.owner + (int64_t)bh * RS;
  const int page0 = bh * RS;
  const int T = min(max(a.seq_lens[b], 0), MB * a.bs);
  for (int s = threadIdx.x; s < RS; s += kRetrieveThreads) fresh[s] = 0;
  if (threadIdx.x == 0) n_ref = 0;

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
  int n_free;
  int base = workgroup_offset(nf, wave_tot, &n_free);
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
      fresh[s] = 1;
    }
    if (hp < 0) flag_error(t.err);
    src_page[j] = hp < 0 ? -1 : hp;
    dst_page[j] = hp < 0 ? -1 : dp;
  }
  __syncthreads();
  // resident pages that took appended tokens in host memory
  const int lo = a.seq_prev ? max(a.seq_prev[b], 0) : -1;
  plan_refresh(t, bh, T, lo, a.bs, res, fresh, page0, RS, nl, src_page, dst_page, rng, &n_ref);
  __syncthreads();

  // 4. copy
  copy_pages(a.hk, a.hv, a.he, a.dk, a.dv, a.de, a.bs * a.D / 8, a.bs / 4, nl, src_page, dst_page);
  refresh_tokens(a.hk, a.hv, a.he, a.dk, a.dv, a.de, a.bs, a.D, nl, n_ref, src_page, dst_page, rng);
}

// ---------------------------------------------------------------------------
// Retrieve with a locality-aware buffer.
//
// Spin summary, 2.B: the GPU buffer of a request holds the pages the step
// needs and buffered pages kept for temporal locality; buffered pages are
// evicted by a bucketed LRU (pages grouped by recency timestamp into, e.g.,
// 64 buckets) decided in parallel on the GPU, with no global sort.
//
// Here a slot's timestamp is the step at which its block was last selected.
// One workgroup per (b, h):
//   1. selected blocks already in a slot are hits (timestamp := step); the
//      others are misses, listed in selection order;
//   2. if the free slots are too few, the buffered pages (resident, not
//      selected) are binned by recency bucket min((age - 1) / width, 63) in
//      an LDS histogram; a wave scan from the oldest bucket finds the bucket
//      where eviction stops; every older page goes, and inside that bucket
//      the lowest slots go first (a workgroup prefix sum of the per-thread
//      counts);
//   3. the j-th miss takes the j-th free slot (ascending), timestamp :=
//      step, and its pages are copied from host memory; appended tokens
//      reach resident pages as in retrieve_kernel.
// ---------------------------------------------------------------------------

struct BufferArgs {
  Table host;
  const uint4* hk;
  const uint4* hv;
  const uint4* he;
  uint4* dk;
  uint4* dv;
  uint4* de;
  int RS, bs, D, cap, step, width;
  int32_t* resident;  // [B][Hkv][max_blocks]
  int32_t* owner;     // [B][Hkv][RS]
  int32_t* last_use;  // [B][Hkv][RS]
  const int32_t* sel;
  const int32_t* sel_count;
  const int32_t* seq_lens;
  const int32_t* seq_prev;  // [B] or null
  int32_t* miss_count;      // [B][Hkv] or null
};

__global__ __launch_bounds__(kRetrieveThreads) void retrieve_buffered_kernel(const BufferArgs a) {
  __shared__ int32_t free_slot[kMaxRetrieveSlots];
  __shared__ int32_t miss[kMaxRetrieveSlots];
  __shared__ int64_t src_page[kMaxRetrieveSlots + 1];
  __shared__ int32_t dst_page[kMaxRetrieveSlots + 1];
  __shared__ uint8_t hit[kMaxRetrieveSlots];
  __shared__ int32_t hist[kRecencyBuckets];
  __shared__ int32_t wave_tot[kRetrieveThreads / kWave];
  __shared__ int32_t rng[kMaxRetrieveSlots + 1];
  __shared__ uint8_t fresh[kMaxRetrieveSlots];
  __shared__ int32_t n_ref, cut_bucket, cut_take;
  const Table& t = a.host;
  const int bh = blockIdx.x;
  const int b = bh / t.Hkv;
  const int MB = t.max_blocks, RS = a.RS, now = a.step;
  int32_t* res = a.resident + (int64_t)bh * MB;
  int32_t* own = a.owner + (int64_t)bh * RS;
  int32_t* lu = a.last_use + (int64_t)bh * RS;
  const int page0 = bh * RS;
  const int T = min(max(a.seq_lens[b], 0), MB * a.bs);
  for (int s = threadIdx.x; s < RS; s += kRetrieveThreads) {
    hit[s] = 0;
    fresh[s] = 0;
  }
  if (threadIdx.x < kRecencyBuckets) hist[threadIdx.x] = 0;
  if (threadIdx.x == 0) n_ref = 0;
  __syncthreads();

  // 1. hits and misses; thread t takes selection entries [4t, 4t + 4)
  //    (sel_count <= cap <= RS <= 4 * 256)
  const int n = min(max(a.sel_count[bh], 0), a.cap);
  int mx[4], nm = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * threadIdx.x + j;
    mx[j] = -1;
    if (i < n) {
      const int x = a.sel[(int64_t)bh * a.cap + i];
      if (x < 0 || x >= MB) {
        flag_error(t.err);
        continue;
      }
      const int p = res[x];
      if (p >= page0 && p < page0 + RS) {
        hit[p - page0] = 1;
        lu[p - page0] = now;
      } else {
        mx[j] = x;
        ++nm;
      }
    }
  }
  int n_miss;
  int base = workgroup_offset(nm, wave_tot, &n_miss);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (mx[j] >= 0) miss[base++] = mx[j];
  }
  __syncthreads();  // hit[] complete

  // 2. slot classes: free (-1), needed this step (-2), or buffered (its
  //    recency bucket); thread t takes slots [4t, 4t + 4)
  int cls[4], nf = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = 4 * threadIdx.x + j;
    cls[j] = -2;
    if (s < RS) {
      const int o = own[s];
      if (o < 0) {
        cls[j] = -1;
        ++nf;
      } else if (!hit[s]) {
        const int age = max(now - lu[s], 1);
        cls[j] = min((age - 1) / a.width, kRecencyBuckets - 1);
      }
    }
  }
  int n_free;
  (void)workgroup_offset(nf, wave_tot, &n_free);
  const int need = n_miss - n_free;  // workgroup-uniform
  bool gone[4] = {false, false, false, false};
  if (need > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (cls[j] >= 0) atomicAdd(&hist[cls[j]], 1);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      // lane L holds bucket 63 - L: the inclusive scan counts the pages of
      // the L + 1 oldest buckets
      const int v = hist[kRecencyBuckets - 1 - threadIdx.x];
      const int incl = wave_scan_incl(v);
      const uint64_t reach = __ballot(incl >= need);
      // the first lane whose count reaches `need` (wave-uniform); none:
      // fewer buffered pages than needed, and all of them go
      const int L = reach != 0 ? (int)__builtin_ctzll(reach) : -1;
      const int before = __builtin_amdgcn_readlane(incl - v, L >= 0 ? L : 0);  // pages in older buckets
      if (threadIdx.x == 0) {
        cut_bucket = L >= 0 ? kRecencyBuckets - 1 - L : -1;
        cut_take = L >= 0 ? need - before : 0;
      }
    }
    __syncthreads();
    const int cb = cut_bucket, take = cut_take;
    int in_cut = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) in_cut += cls[j] >= 0 && cls[j] == cb;
    int total_cut;
    int rank = workgroup_offset(in_cut, wave_tot, &total_cut);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (cls[j] < 0) continue;
      if (cls[j] > cb) {
        gone[j] = true;
      } else if (cls[j] == cb) {
        gone[j] = rank < take;
        ++rank;
      }
      if (gone[j]) {
        const int s = 4 * threadIdx.x + j;
        const int x = own[s];
        if (x >= 0 && x < MB) res[x] = -1;
        own[s] = -1;
      }
    }
  }

  // 3. the free slots (old and just freed) in ascending order
  int fr = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) fr += cls[j] == -1 || gone[j];
  int n_avail;
  base = workgroup_offset(fr, wave_tot, &n_avail);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (cls[j] == -1 || gone[j]) free_slot[base++] = 4 * threadIdx.x + j;
  }
  __syncthreads();

  // 4. misses take the free slots in order
  int nl = n_miss;
  if (nl > n_avail) {
    if (threadIdx.x == 0) flag_error(t.err);
    nl = n_avail;
  }
  for (int j = threadIdx.x; j < nl; j += kRetrieveThreads) {
    const int y = miss[j];
    uint32_t doc;
    const int64_t hp = page_of_any(t, bh, y, doc);
    const int s = free_slot[j];
    own[s] = y;
    res[y] = page0 + s;
    lu[s] = now;
    fresh[s] = 1;
    if (hp < 0) flag_error(t.err);
    src_page[j] = hp < 0 ? -1 : hp;
    dst_page[j] = hp < 0 ? -1 : page0 + s;
  }
  if (threadIdx.x == 0 && a.miss_count) a.miss_count[bh] = nl;
  __syncthreads();
  const int lo = a.seq_prev ? max(a.seq_prev[b], 0) : -1;
  plan_refresh(t, bh, T, lo, a.bs, res, fresh, page0, RS, nl, src_page, dst_page, rng, &n_ref);
  __syncthreads();

  // 5. copy
  copy_pages(a.hk, a.hv, a.he, a.dk, a.dv, a.de, a.bs * a.D / 8, a.bs / 4, nl, src_page, dst_page);
  refresh_tokens(a.hk, a.hv, a.he, a.dk, a.dv, a.de, a.bs, a.D, nl, n_ref, src_page, dst_page, rng);
}

hipError_t launch_retrieve(const nosa_dims& d, const nosa_kv& host_kv, const void* host_k, const void* host_v,
                           const void* host_e, uint16_t* dev_k, uint16_t* dev_v, float* dev_e, int32_t slots,
                           int32_t* resident, int32_t* slot_owner, const int32_t* load, const int32_t* load_count,
                           const int32_t* evict, const int32_t* evict_count, int32_t cap, const int32_t* seq_lens,
                           const int32_t* seq_prev, hipStream_t stream) {
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
  a.seq_prev = seq_prev;
  retrieve_kernel<<<d.batch * d.n_kv_heads, kRetrieveThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_retrieve_buffered(const nosa_dims& d, const nosa_kv& host_kv, const void* host_k,
                                    const void* host_v, const void* host_e, uint16_t* dev_k, uint16_t* dev_v,
                                    float* dev_e, int32_t slots, int32_t* resident, int32_t* slot_owner,
                                    int32_t* last_use, const int32_t* sel, const int32_t* sel_count, int32_t cap,
                                    int32_t step, int32_t bucket_width, const int32_t* seq_lens,
                                    const int32_t* seq_prev, int32_t* miss_count, hipStream_t stream) {
  BufferArgs a;
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
  a.step = step;
  a.width = bucket_width;
  a.resident = resident;
  a.owner = slot_owner;
  a.last_use = last_use;
  a.sel = sel;
  a.sel_count = sel_count;
  a.seq_lens = seq_lens;
  a.seq_prev = seq_prev;
  a.miss_count = miss_count;
  retrieve_buffered_kernel<<<d.batch * d.n_kv_heads, kRetrieveThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace nosa
