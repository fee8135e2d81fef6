// Bandwidth probes: what the HBM gives this GPU for the step's two access
// patterns when nothing is computed on the data.  They are measurement
// tools, not part of the step, and give the practical ceilings the step's
// kernels are compared with:
//   * stream_read_kernel: a contiguous buffer read once with 16-byte
//     non-temporal loads -- the pattern of the block-summary stream that
//     the scoring reads;
//   * page_gather_kernel: the K page and the V page of every listed page id
//     read whole -- the selected-page gather of the decode, with its grid
//     (one workgroup of four waves per list, one list per (b, h) pair, wave
//     w taking pages w, w + 4, ...), its loads (16-byte non-temporal) and its
//     bytes in flight per wave (the next K page while the V page lands).
// Every workgroup folds what it read into one 32-bit word (xor of all
// words), written to sink[workgroup], so no load can be dropped and the host
// can check that every byte was read.

#include "nosa_device.hpp"
#include "nosa_launch.hpp"

namespace nosa {

constexpr int kProbeThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return v.x ^ v.y ^ v.z ^ v.w;
}

// xor over the workgroup, written by thread 0
__device__ __forceinline__ void sink_workgroup(uint32_t acc, uint32_t* sink) {
  __shared__ uint32_t part[kProbeThreads / kWave];
  acc = xor_reduce<1, kWave>(acc, [](uint32_t x, uint32_t y) { return x ^ y; });
  if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / kWave; ++w) t ^= part[w];
    sink[blockIdx.x] = t;
  }
}

// n16 16-byte units; grid-stride, eight loads in flight per thread.
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* src, int64_t n16,
                                                                    uint32_t* sink) {
  constexpr int U = 8;
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint32_t f[U];
#pragma unroll
    for (int u = 0; u < U; ++u) f[u] = fold_nt(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= f[u];
  }
  for (; i < n16; i += stride) acc ^= fold_nt(src + i);
  sink_workgroup(acc, sink);
}

// Pages of PU 16-byte units per lane (page = kWave * PU units); list
// blockIdx.x holds ppl <= kWaves * kWave page ids, and lane j of wave w holds
// the wave's page w + kWaves * j.  Ids outside [0, num_pages) are skipped.
// The wave streams its pages as half pages (the K page, then the V page)
// through two register buffers: the next half is issued before the current
// one is folded, so one K page and one V page are in flight, as in the
// decode's loop.  Every branch between an issue and its fold is uniform and
// each path is straight-line code, so each fold waits for its own loads only.
template <int PU>
__global__ __launch_bounds__(kProbeThreads, 1) void page_gather_kernel(const uint4* k_pool, const uint4* v_pool,
                                                                       int64_t num_pages, const int32_t* pages,
                                                                       int ppl, uint32_t* sink) {
  constexpr int kWaves = kProbeThreads / kWave;
  constexpr int64_t kPage = (int64_t)kWave * PU;  // 16-byte units per page
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int32_t* list = pages + (int64_t)blockIdx.x * ppl;
  const int slot = w + kWaves * lane;
  const int32_t mine = slot < ppl ? list[slot] : -1;
  uint64_t rest = __ballot(mine >= 0 && mine < num_pages);  // this wave's pages still to issue
  uint32_t acc = 0;
  uint4 a[PU], b[PU];
  int32_t pg = 0;
  int part = 2;  // half of page pg issued last: 0 = K, 1 = V (2: none yet)
  // the next half page, or nullptr when the wave has issued them all
  auto next_half = [&]() -> const uint4* {
    if (part == 0) {
      part = 1;
      return v_pool + pg * kPage + lane;
    }
    if (rest == 0) return nullptr;
    pg = __builtin_amdgcn_readlane(mine, __ffsll((unsigned long long)rest) - 1);
    rest &= rest - 1;
    part = 0;
    return k_pool + pg * kPage + lane;
  };
  auto load = [&](uint4 (&buf)[PU], const uint4* src) {
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + u * kWave));
      buf[u] = make_uint4(v.x, v.y, v.z, v.w);
    }
  };
  auto fold = [&](const uint4 (&buf)[PU]) {
#pragma unroll
    for (int u = 0; u < PU; ++u) acc ^= buf[u].x ^ buf[u].y ^ buf[u].z ^ buf[u].w;
  };
  const uint4* src = next_half();
  if (src != nullptr) {
    load(a, src);
    while (true) {
      src = next_half();
      if (src == nullptr) {
        fold(a);
        break;
      }
      load(b, src);
      fold(a);
      src = next_half();
      if (src == nullptr) {
        fold(b);
        break;
      }
      load(a, src);
      fold(b);
    }
  }
  sink_workgroup(acc, sink);
}

hipError_t launch_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t n_workgroups,
                                    hipStream_t stream) {
  stream_read_kernel<<<n_workgroups, kProbeThreads, 0, stream>>>(reinterpret_cast<const uint4*>(src), bytes / 16,
                                                                  sink);
  return hipGetLastError();
}

hipError_t launch_probe_page_gather(const void* k_pool, const void* v_pool, int64_t page_bytes, int64_t num_pages,
                                    const int32_t* pages, int32_t n_lists, int32_t pages_per_list, uint32_t* sink,
                                    hipStream_t stream) {
  const uint4* kp = reinterpret_cast<const uint4*>(k_pool);
  const uint4* vp = reinterpret_cast<const uint4*>(v_pool);
  switch (page_bytes / (16 * kWave)) {  // 16-byte units per lane
    case 8:
      page_gather_kernel<8><<<n_lists, kProbeThreads, 0, stream>>>(kp, vp, num_pages, pages, pages_per_list, sink);
      break;
    case 16:
      page_gather_kernel<16><<<n_lists, kProbeThreads, 0, stream>>>(kp, vp, num_pages, pages, pages_per_list, sink);
      break;
    default:
      page_gather_kernel<32><<<n_lists, kProbeThreads, 0, stream>>>(kp, vp, num_pages, pages, pages_per_list, sink);
      break;
  }
  return hipGetLastError();
}

}  // namespace nosa
