// Internal launchers, one per kernel family.  Arguments are already checked
// by the C-ABI layer (nosa_api.cpp); each launcher only picks the template
// instance and enqueues the kernel on `stream`.  Host-only declarations (the
// HIP runtime API, no device code), so the C-ABI layer also builds as plain
// C++ with a host compiler.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "nosa.h"

namespace nosa {

constexpr int kMaxRetrieveSlots = 1024;  // resident slots per (b, h) in the host-tier retrieve

hipError_t launch_prefill(const nosa_dims& d, const nosa_kv& kv, const uint16_t* k_src,
                          const uint16_t* v_src, const float* e_src, int32_t src_tokens,
                          const int32_t* seq_lens, hipStream_t stream);

hipError_t launch_build_summaries(const nosa_dims& d, const nosa_kv& kv, const int32_t* seq_lens,
                                  float* k_summary, float* e_summary, hipStream_t stream);

hipError_t launch_append(const nosa_dims& d, const nosa_kv& kv, const uint16_t* k_new,
                         const uint16_t* v_new, const float* e_new, int32_t* seq_lens,
                         float* k_summary, float* e_summary, hipStream_t stream);

hipError_t launch_score(const nosa_dims& d, const uint16_t* q, const float* k_summary,
                        const float* e_summary, const int32_t* seq_lens, float* score_q,
                        float* score_e, hipStream_t stream);

hipError_t launch_select(const nosa_dims& d, const float* score_q, const float* score_e,
                         const int32_t* seq_lens, int32_t k_e, int32_t k_q, uint32_t* evicted,
                         int32_t* sel, int32_t sel_cap, int32_t* sel_count, hipStream_t stream);

hipError_t launch_select_swap(const nosa_dims& d, const float* score_q, const float* score_e,
                              const int32_t* seq_lens, int32_t k_e, int32_t k_q, uint32_t* evicted,
                              int32_t* sel, int32_t sel_cap, int32_t* sel_count, const int32_t* prev,
                              const int32_t* prev_count, int32_t* load, int32_t* load_count, int32_t* evict,
                              int32_t* evict_count, hipStream_t stream);

hipError_t launch_append_score(const nosa_dims& d, const nosa_kv& kv, const uint16_t* k_new,
                               const uint16_t* v_new, const float* e_new, const int32_t* seq_lens_in,
                               int32_t* seq_lens_out, float* k_summary, float* e_summary, const uint16_t* q,
                               float* score_q, float* score_e, hipStream_t stream);

hipError_t launch_swap_diff(const nosa_dims& d, int32_t cap, const int32_t* prev,
                            const int32_t* prev_count, const int32_t* cur, const int32_t* cur_count,
                            int32_t* load, int32_t* load_count, int32_t* evict,
                            int32_t* evict_count, hipStream_t stream);

hipError_t launch_decode(const nosa_dims& d, const uint16_t* q, const nosa_kv& kv,
                         const int32_t* sel, const int32_t* sel_count, int32_t sel_cap,
                         const int32_t* seq_lens, int32_t num_splits, float sm_scale,
                         float* part_o, float* part_m, float* part_l, int32_t* counters, float* o,
                         float* m, float* l, hipStream_t stream);

hipError_t launch_select_decode(const nosa_dims& d, const uint16_t* q, const nosa_kv& kv, const float* score_q,
                                const float* score_e, const int32_t* seq_lens, int32_t k_e, int32_t k_q,
                                const uint32_t* evicted_in, uint32_t* evicted_out, int32_t* sel, int32_t sel_cap,
                                int32_t* sel_count, const int32_t* prev, const int32_t* prev_count, int32_t* load,
                                int32_t* load_count, int32_t* evict, int32_t* evict_count, int32_t num_splits,
                                float sm_scale, float* part_o, float* part_m, float* part_l, int32_t* counters,
                                float* o, float* m, float* l, hipStream_t stream);

// Layout of the static scratch of nosa_select_decode_noalloc: the arrival
// counters (one int32 per pair, at most 65535 pairs) first, then the split
// partials part_m, part_l [B*Hq*P] and part_o [B*Hq*P*D] fp32, each on a
// 256-byte boundary.
constexpr int64_t kNoAllocScratchBytes = NOSA_NOALLOC_SCRATCH_BYTES;
constexpr int64_t kNoAllocCountersOffset = 0;
constexpr int64_t kNoAllocCountersBytes = 65536 * 4;

struct NoAllocLayout {
  int64_t part_m, part_l, part_o, total;
};

inline NoAllocLayout noalloc_layout(const nosa_dims& d, int32_t num_splits) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t rows = (int64_t)d.batch * d.n_q_heads * num_splits;
  NoAllocLayout lay;
  lay.part_m = kNoAllocCountersOffset + kNoAllocCountersBytes;
  lay.part_l = lay.part_m + up(rows * 4);
  lay.part_o = lay.part_l + up(rows * 4);
  lay.total = lay.part_o + up(rows * d.head_dim * 4);
  return lay;
}

hipError_t launch_select_decode_noalloc(const nosa_dims& d, const uint16_t* q, const nosa_kv& kv,
                                        const float* score_q, const float* score_e, const int32_t* seq_lens,
                                        int32_t k_e, int32_t k_q, const uint32_t* evicted_in, uint32_t* evicted_out,
                                        int32_t* sel, int32_t sel_cap, int32_t* sel_count, const int32_t* prev,
                                        const int32_t* prev_count, int32_t* load, int32_t* load_count,
                                        int32_t* evict, int32_t* evict_count, int32_t num_splits, float sm_scale,
                                        float* o, float* m, float* l, hipStream_t stream);

hipError_t launch_retrieve(const nosa_dims& d, const nosa_kv& host_kv, const void* host_k, const void* host_v,
                           const void* host_e, uint16_t* dev_k, uint16_t* dev_v, float* dev_e, int32_t slots,
                           int32_t* resident, int32_t* slot_owner, const int32_t* load, const int32_t* load_count,
                           const int32_t* evict, const int32_t* evict_count, int32_t cap, const int32_t* seq_lens,
                           const int32_t* seq_prev, hipStream_t stream);

hipError_t launch_retrieve_buffered(const nosa_dims& d, const nosa_kv& host_kv, const void* host_k,
                                    const void* host_v, const void* host_e, uint16_t* dev_k, uint16_t* dev_v,
                                    float* dev_e, int32_t slots, int32_t* resident, int32_t* slot_owner,
                                    int32_t* last_use, const int32_t* sel, const int32_t* sel_count, int32_t cap,
                                    int32_t step, int32_t bucket_width, const int32_t* seq_lens,
                                    const int32_t* seq_prev, int32_t* miss_count, hipStream_t stream);

hipError_t launch_decode_mass(const nosa_dims& d, const uint16_t* q, const nosa_kv& kv, const int32_t* sel,
                              const int32_t* sel_count, int32_t sel_cap, const int32_t* seq_lens, int32_t num_splits,
                              float sm_scale, float* part_o, float* part_m, float* part_l, int32_t* counters, float* o,
                              float* m, float* l, float* tile_stats, float* mass, hipStream_t stream);

hipError_t launch_decode_alibi(const nosa_dims& d, const uint16_t* q, const nosa_kv& kv, const int32_t* sel,
                               const int32_t* sel_count, int32_t sel_cap, const int32_t* seq_lens,
                               int32_t num_splits, float sm_scale, const float* alibi_slopes, float* part_o,
                               float* part_m, float* part_l, int32_t* counters, float* o, float* m, float* l,
                               hipStream_t stream);

hipError_t launch_append_score_qkv(const nosa_dims& d, const nosa_kv& kv, const uint16_t* qkv, const float* w_evict,
                                   const int32_t* seq_lens_in, int32_t* seq_lens_out, float* k_summary,
                                   float* e_summary, uint16_t* q_out, float* score_q, float* score_e,
                                   hipStream_t stream);

hipError_t launch_prefill_attention(const nosa_dims& d, const nosa_kv& kv, const uint16_t* q, int32_t n_prompt,
                                    const int32_t* q_pos0, const int32_t* seq_lens, float sm_scale, float* o,
                                    float* m, float* l, hipStream_t stream);

hipError_t launch_combine(const nosa_dims& d, int32_t num_splits, const float* part_o,
                          const float* part_m, const float* part_l, float* o, float* m, float* l,
                          hipStream_t stream);

hipError_t launch_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t n_workgroups,
                                    hipStream_t stream);

hipError_t launch_probe_page_gather(const void* k_pool, const void* v_pool, int64_t page_bytes, int64_t num_pages,
                                    const int32_t* pages, int32_t n_lists, int32_t pages_per_list, uint32_t* sink,
                                    hipStream_t stream);

}  // namespace nosa
