// C-ABI entry points of libnosa: argument checks, then one launch each.
// The checks are plain host logic and touch no HIP API, so a failing call
// returns before anything is enqueued.

#include <stdint.h>

#include "nosa.h"
#include "nosa_launch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

nosa_status check_dims(const nosa_dims* d) {
  if (!d) return NOSA_ERR_ARG;
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 || d->block_size < 1 ||
      d->sub_block < 1 || d->max_blocks < 1)
    return NOSA_ERR_ARG;
  if (d->n_q_heads % d->n_kv_heads != 0) return NOSA_ERR_ARG;
  if (d->block_size % d->sub_block != 0) return NOSA_ERR_ARG;
  if ((int64_t)d->batch * d->n_kv_heads > 65535) return NOSA_ERR_UNSUPPORTED;
  if ((int64_t)d->batch * d->n_q_heads > (int64_t)1 << 30) return NOSA_ERR_UNSUPPORTED;
  const int G = d->n_q_heads / d->n_kv_heads;
  if (!pow2(G) || G > 16) return NOSA_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return NOSA_ERR_UNSUPPORTED;
  if (d->block_size != 64 && d->block_size != 128 && d->block_size != 256) return NOSA_ERR_UNSUPPORTED;
  const int nsub = d->block_size / d->sub_block;
  if (!pow2(nsub) || nsub > 64) return NOSA_ERR_UNSUPPORTED;
  if (d->max_blocks > 8192) return NOSA_ERR_UNSUPPORTED;
  return NOSA_OK;
}

// `need_pages`: the call reads or writes the page pools.
nosa_status check_kv(const nosa_dims* d, const nosa_kv* kv, bool need_pages) {
  if (!kv) return NOSA_ERR_ARG;
  if (kv->num_pages < 1) return NOSA_ERR_ARG;
  if (need_pages) {
    if (!kv->k_pages || !kv->v_pages || !kv->e_pages) return NOSA_ERR_ARG;
    if (!aligned16(kv->k_pages) || !aligned16(kv->v_pages) || !aligned16(kv->e_pages)) return NOSA_ERR_ARG;
  }
  switch (kv->kind) {
    case NOSA_TABLE_FLAT:
      if (!kv->table) return NOSA_ERR_ARG;
      break;
    case NOSA_TABLE_TWO_LEVEL: {
      if (!kv->directory || !kv->segments || kv->num_segments < 1) return NOSA_ERR_ARG;
      if (kv->seg_log2 < 0 || kv->seg_log2 > 20 || kv->blocks_log2 < kv->seg_log2 || kv->blocks_log2 > 24)
        return NOSA_ERR_ARG;
      if ((int64_t)d->max_blocks > ((int64_t)1 << kv->blocks_log2)) return NOSA_ERR_ARG;
      const int64_t need = (((int64_t)d->batch * d->n_kv_heads) << kv->blocks_log2) >> kv->seg_log2;
      if ((int64_t)kv->dir_entries < need) return NOSA_ERR_ARG;
      break;
    }
    case NOSA_TABLE_PACKED_ROPE:
      if (!kv->packed) return NOSA_ERR_ARG;
      if (kv->num_pages > ((int64_t)1 << NOSA_PACK_PAGE_BITS)) return NOSA_ERR_ARG;
      break;
    default:
      return NOSA_ERR_ARG;
  }
  return NOSA_OK;
}

nosa_status from_hip(hipError_t e) { return e == hipSuccess ? NOSA_OK : NOSA_ERR_HIP; }

}  // namespace

extern "C" {

nosa_status nosa_prefill_pages(const nosa_dims* dims, const nosa_kv* kv, const uint16_t* k_src,
                               const uint16_t* v_src, const float* e_src, int32_t src_tokens,
                               const int32_t* seq_lens, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, kv, true)) != NOSA_OK) return st;
  if (!k_src || !v_src || !e_src || !seq_lens || src_tokens < 0) return NOSA_ERR_ARG;
  if (!aligned16(k_src)) return NOSA_ERR_ARG;
  return from_hip(nosa::launch_prefill(*dims, *kv, k_src, v_src, e_src, src_tokens, seq_lens, stream));
}

nosa_status nosa_build_summaries(const nosa_dims* dims, const nosa_kv* kv, const int32_t* seq_lens,
                                 float* k_summary, float* e_summary, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, kv, true)) != NOSA_OK) return st;
  if (!seq_lens || !k_summary || !e_summary || !aligned16(k_summary)) return NOSA_ERR_ARG;
  return from_hip(nosa::launch_build_summaries(*dims, *kv, seq_lens, k_summary, e_summary, stream));
}

nosa_status nosa_append(const nosa_dims* dims, const nosa_kv* kv, const uint16_t* k_new,
                        const uint16_t* v_new, const float* e_new, int32_t* seq_lens, float* k_summary,
                        float* e_summary, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, kv, true)) != NOSA_OK) return st;
  if (!k_new || !v_new || !e_new || !seq_lens || !k_summary || !e_summary) return NOSA_ERR_ARG;
  if (!aligned16(k_new) || !aligned16(k_summary)) return NOSA_ERR_ARG;
  if (dims->n_kv_heads > 16) return NOSA_ERR_UNSUPPORTED;
  return from_hip(
      nosa::launch_append(*dims, *kv, k_new, v_new, e_new, seq_lens, k_summary, e_summary, stream));
}

nosa_status nosa_score_blocks(const nosa_dims* dims, const uint16_t* q, const float* k_summary,
                              const float* e_summary, const int32_t* seq_lens, float* score_q,
                              float* score_e, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if (!q || !k_summary || !e_summary || !seq_lens || !score_q || !score_e) return NOSA_ERR_ARG;
  if (!aligned16(k_summary)) return NOSA_ERR_ARG;
  return from_hip(nosa::launch_score(*dims, q, k_summary, e_summary, seq_lens, score_q, score_e, stream));
}

nosa_status nosa_select(const nosa_dims* dims, const float* score_q, const float* score_e,
                        const int32_t* seq_lens, int32_t k_e, int32_t k_q, uint32_t* evicted, int32_t* sel,
                        int32_t sel_cap, int32_t* sel_count, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if (!score_q || !score_e || !seq_lens || !evicted || !sel || !sel_count) return NOSA_ERR_ARG;
  if (k_e < 0 || k_q < 0 || sel_cap < 1) return NOSA_ERR_ARG;
  const int64_t k = (int64_t)k_e + k_q;
  if ((int64_t)sel_cap < (k < dims->max_blocks ? k : (int64_t)dims->max_blocks)) return NOSA_ERR_ARG;
  return from_hip(
      nosa::launch_select(*dims, score_q, score_e, seq_lens, k_e, k_q, evicted, sel, sel_cap, sel_count, stream));
}

nosa_status nosa_select_swap(const nosa_dims* dims, const float* score_q, const float* score_e,
                             const int32_t* seq_lens, int32_t k_e, int32_t k_q, uint32_t* evicted, int32_t* sel,
                             int32_t sel_cap, int32_t* sel_count, const int32_t* prev, const int32_t* prev_count,
                             int32_t* load, int32_t* load_count, int32_t* evict, int32_t* evict_count,
                             hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if (!score_q || !score_e || !seq_lens || !evicted || !sel || !sel_count) return NOSA_ERR_ARG;
  if (!prev || !prev_count || !load || !load_count || !evict || !evict_count) return NOSA_ERR_ARG;
  if (k_e < 0 || k_q < 0 || sel_cap < 1) return NOSA_ERR_ARG;
  const int64_t k = (int64_t)k_e + k_q;
  if ((int64_t)sel_cap < (k < dims->max_blocks ? k : (int64_t)dims->max_blocks)) return NOSA_ERR_ARG;
  if (sel_cap > dims->max_blocks) return NOSA_ERR_ARG;
  if (prev == sel || load == sel || evict == sel || load == evict) return NOSA_ERR_ARG;
  return from_hip(nosa::launch_select_swap(*dims, score_q, score_e, seq_lens, k_e, k_q, evicted, sel, sel_cap,
                                           sel_count, prev, prev_count, load, load_count, evict, evict_count,
                                           stream));
}

nosa_status nosa_append_score(const nosa_dims* dims, const nosa_kv* kv, const uint16_t* k_new,
                              const uint16_t* v_new, const float* e_new, const int32_t* seq_lens_in,
                              int32_t* seq_lens_out, float* k_summary, float* e_summary, const uint16_t* q,
                              float* score_q, float* score_e, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  const bool append = k_new != nullptr;
  if ((st = check_kv(dims, kv, append)) != NOSA_OK) return st;
  if (append) {
    if (!v_new || !e_new || !seq_lens_out || !aligned16(k_new)) return NOSA_ERR_ARG;
    if (seq_lens_out == seq_lens_in) return NOSA_ERR_ARG;
  } else if (v_new || e_new) {
    return NOSA_ERR_ARG;
  }
  if (!seq_lens_in || !k_summary || !e_summary || !q || !score_q || !score_e) return NOSA_ERR_ARG;
  if (!aligned16(k_summary)) return NOSA_ERR_ARG;
  if (kv->kind == NOSA_TABLE_PACKED_ROPE) {  // scoring with the rotated query; no append
    if (append) return NOSA_ERR_UNSUPPORTED;
    if (!kv->q_pos || !(kv->rope_base > 1.f)) return NOSA_ERR_ARG;
    const int nsub = dims->block_size / dims->sub_block;
    if (nsub < 4 || nsub > 16) return NOSA_ERR_UNSUPPORTED;
  }
  return from_hip(nosa::launch_append_score(*dims, *kv, k_new, v_new, e_new, seq_lens_in, seq_lens_out, k_summary,
                                            e_summary, q, score_q, score_e, stream));
}

nosa_status nosa_append_score_qkv(const nosa_dims* dims, const nosa_kv* kv, const uint16_t* qkv,
                                  const float* w_evict, const int32_t* seq_lens_in, int32_t* seq_lens_out,
                                  float* k_summary, float* e_summary, uint16_t* q_out, float* score_q,
                                  float* score_e, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, kv, true)) != NOSA_OK) return st;
  if (kv->kind == NOSA_TABLE_PACKED_ROPE) return NOSA_ERR_UNSUPPORTED;
  if (!qkv || !w_evict || !seq_lens_in || !seq_lens_out || !k_summary || !e_summary || !q_out || !score_q ||
      !score_e)
    return NOSA_ERR_ARG;
  if (seq_lens_out == seq_lens_in) return NOSA_ERR_ARG;
  if (!aligned16(qkv) || !aligned16(q_out) || !aligned16(k_summary)) return NOSA_ERR_ARG;
  return from_hip(nosa::launch_append_score_qkv(*dims, *kv, qkv, w_evict, seq_lens_in, seq_lens_out, k_summary,
                                                e_summary, q_out, score_q, score_e, stream));
}

nosa_status nosa_swap_diff(const nosa_dims* dims, int32_t cap, const int32_t* prev, const int32_t* prev_count,
                           const int32_t* cur, const int32_t* cur_count, int32_t* load, int32_t* load_count,
                           int32_t* evict, int32_t* evict_count, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if (cap < 1 || !prev || !prev_count || !cur || !cur_count || !load || !load_count || !evict || !evict_count)
    return NOSA_ERR_ARG;
  return from_hip(nosa::launch_swap_diff(*dims, cap, prev, prev_count, cur, cur_count, load, load_count, evict,
                                         evict_count, stream));
}

nosa_status nosa_sparse_decode(const nosa_dims* dims, const uint16_t* q, const nosa_kv* kv, const int32_t* sel,
                               const int32_t* sel_count, int32_t sel_cap, const int32_t* seq_lens,
                               int32_t num_splits, float sm_scale, float* part_o, float* part_m,
                               float* part_l, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, kv, true)) != NOSA_OK) return st;
  if (!q || !sel || !sel_count || !seq_lens || !part_o || !part_m || !part_l) return NOSA_ERR_ARG;
  if (!aligned16(q)) return NOSA_ERR_ARG;
  if (sel_cap < 1 || num_splits < 1 || num_splits > 256) return NOSA_ERR_ARG;
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return NOSA_ERR_ARG;
  if (kv->kind == NOSA_TABLE_PACKED_ROPE) {
    if (!kv->q_pos || !(kv->rope_base > 1.f)) return NOSA_ERR_ARG;
    if (dims->n_q_heads / dims->n_kv_heads > 8) return NOSA_ERR_UNSUPPORTED;
  }
  return from_hip(nosa::launch_decode(*dims, q, *kv, sel, sel_count, sel_cap, seq_lens, num_splits, sm_scale,
                                      part_o, part_m, part_l, nullptr, nullptr, nullptr, nullptr, stream));
}

nosa_status nosa_sparse_decode_combine(const nosa_dims* dims, const uint16_t* q, const nosa_kv* kv,
                                       const int32_t* sel, const int32_t* sel_count, int32_t sel_cap,
                                       const int32_t* seq_lens, int32_t num_splits, float sm_scale,
                                       float* part_o, float* part_m, float* part_l, int32_t* counters,
                                       float* o, float* m, float* l, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, kv, true)) != NOSA_OK) return st;
  if (!q || !sel || !sel_count || !seq_lens || !part_o || !part_m || !part_l) return NOSA_ERR_ARG;
  if (!counters || !o || !m || !l) return NOSA_ERR_ARG;
  if (!aligned16(q)) return NOSA_ERR_ARG;
  if (sel_cap < 1 || num_splits < 1 || num_splits > 256) return NOSA_ERR_ARG;
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return NOSA_ERR_ARG;
  if (kv->kind == NOSA_TABLE_PACKED_ROPE) {
    if (!kv->q_pos || !(kv->rope_base > 1.f)) return NOSA_ERR_ARG;
    if (dims->n_q_heads / dims->n_kv_heads > 8) return NOSA_ERR_UNSUPPORTED;
  }
  return from_hip(nosa::launch_decode(*dims, q, *kv, sel, sel_count, sel_cap, seq_lens, num_splits, sm_scale,
                                      part_o, part_m, part_l, counters, o, m, l, stream));
}

nosa_status nosa_sparse_decode_mass(const nosa_dims* dims, const uint16_t* q, const nosa_kv* kv,
                                    const int32_t* sel, const int32_t* sel_count, int32_t sel_cap,
                                    const int32_t* seq_lens, int32_t num_splits, float sm_scale, float* part_o,
                                    float* part_m, float* part_l, int32_t* counters, float* o, float* m, float* l,
                                    float* tile_stats, float* mass, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, kv, true)) != NOSA_OK) return st;
  if (!q || !sel || !sel_count || !seq_lens || !part_o || !part_m || !part_l) return NOSA_ERR_ARG;
  if (!counters || !o || !m || !l || !tile_stats || !mass) return NOSA_ERR_ARG;
  if (!aligned16(q)) return NOSA_ERR_ARG;
  if (sel_cap < 1 || num_splits < 1 || num_splits > 256) return NOSA_ERR_ARG;
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return NOSA_ERR_ARG;
  if (kv->kind == NOSA_TABLE_PACKED_ROPE) return NOSA_ERR_UNSUPPORTED;
  return from_hip(nosa::launch_decode_mass(*dims, q, *kv, sel, sel_count, sel_cap, seq_lens, num_splits, sm_scale,
                                           part_o, part_m, part_l, counters, o, m, l, tile_stats, mass, stream));
}

nosa_status nosa_sparse_decode_alibi(const nosa_dims* dims, const uint16_t* q, const nosa_kv* kv,
                                     const int32_t* sel, const int32_t* sel_count, int32_t sel_cap,
                                     const int32_t* seq_lens, int32_t num_splits, float sm_scale,
                                     const float* alibi_slopes, float* part_o, float* part_m, float* part_l,
                                     int32_t* counters, float* o, float* m, float* l, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, kv, true)) != NOSA_OK) return st;
  if (!q || !sel || !sel_count || !seq_lens || !part_o || !part_m || !part_l || !alibi_slopes) return NOSA_ERR_ARG;
  if (!counters || !o || !m || !l) return NOSA_ERR_ARG;
  if (!aligned16(q)) return NOSA_ERR_ARG;
  if (sel_cap < 1 || num_splits < 1 || num_splits > 256) return NOSA_ERR_ARG;
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return NOSA_ERR_ARG;
  if (kv->kind == NOSA_TABLE_PACKED_ROPE) return NOSA_ERR_UNSUPPORTED;
  return from_hip(nosa::launch_decode_alibi(*dims, q, *kv, sel, sel_count, sel_cap, seq_lens, num_splits, sm_scale,
                                            alibi_slopes, part_o, part_m, part_l, counters, o, m, l, stream));
}

nosa_status nosa_prefill_attention(const nosa_dims* dims, const nosa_kv* kv, const uint16_t* q, int32_t n_prompt,
                                   const int32_t* q_pos0, const int32_t* seq_lens, float sm_scale, float* o,
                                   float* m, float* l, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, kv, false)) != NOSA_OK) return st;
  if (kv->kind != NOSA_TABLE_PACKED_ROPE) return NOSA_ERR_UNSUPPORTED;
  if (!(kv->rope_base > 1.f)) return NOSA_ERR_ARG;
  if (!q || !q_pos0 || !seq_lens || !o || !m || !l || n_prompt < 1 || !aligned16(q)) return NOSA_ERR_ARG;
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return NOSA_ERR_ARG;
  if ((dims->block_size % 64) != 0) return NOSA_ERR_UNSUPPORTED;
  if ((int64_t)dims->batch * n_prompt * dims->n_q_heads * dims->head_dim > ((int64_t)1 << 40)) return NOSA_ERR_ARG;
  return from_hip(nosa::launch_prefill_attention(*dims, *kv, q, n_prompt, q_pos0, seq_lens, sm_scale, o, m, l,
                                                 stream));
}

nosa_status nosa_select_decode(const nosa_dims* dims, const nosa_kv* kv, const uint16_t* q, const float* score_q,
                               const float* score_e, const int32_t* seq_lens, int32_t k_e, int32_t k_q,
                               const uint32_t* evicted_in, uint32_t* evicted_out, int32_t* sel, int32_t sel_cap,
                               int32_t* sel_count, const int32_t* prev, const int32_t* prev_count, int32_t* load,
                               int32_t* load_count, int32_t* evict, int32_t* evict_count, int32_t num_splits,
                               float sm_scale, float* part_o, float* part_m, float* part_l, int32_t* counters,
                               float* o, float* m, float* l, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, kv, true)) != NOSA_OK) return st;
  if (dims->max_blocks > NOSA_SELECT_DECODE_MAX_BLOCKS) return NOSA_ERR_UNSUPPORTED;
  if (kv->kind == NOSA_TABLE_PACKED_ROPE) {
    if (!kv->q_pos || !(kv->rope_base > 1.f)) return NOSA_ERR_ARG;
    if (dims->n_q_heads / dims->n_kv_heads > 8) return NOSA_ERR_UNSUPPORTED;
  }
  if (!q || !score_q || !score_e || !seq_lens || !evicted_in || !evicted_out || !sel || !sel_count)
    return NOSA_ERR_ARG;
  if (!prev || !prev_count || !load || !load_count || !evict || !evict_count) return NOSA_ERR_ARG;
  if (!part_o || !part_m || !part_l || !counters || !o || !m || !l) return NOSA_ERR_ARG;
  if (!aligned16(q)) return NOSA_ERR_ARG;
  if (k_e < 0 || k_q < 0 || sel_cap < 1 || sel_cap > dims->max_blocks) return NOSA_ERR_ARG;
  const int64_t k = (int64_t)k_e + k_q;
  if ((int64_t)sel_cap < (k < dims->max_blocks ? k : (int64_t)dims->max_blocks)) return NOSA_ERR_ARG;
  if (prev == sel || load == sel || evict == sel || load == evict) return NOSA_ERR_ARG;
  if (num_splits < 1 || num_splits > 256) return NOSA_ERR_ARG;
  if (num_splits > 1 && evicted_in == evicted_out) return NOSA_ERR_ARG;
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return NOSA_ERR_ARG;
  return from_hip(nosa::launch_select_decode(*dims, q, *kv, score_q, score_e, seq_lens, k_e, k_q, evicted_in,
                                             evicted_out, sel, sel_cap, sel_count, prev, prev_count, load, load_count,
                                             evict, evict_count, num_splits, sm_scale, part_o, part_m, part_l,
                                             counters, o, m, l, stream));
}

nosa_status nosa_select_decode_noalloc(const nosa_dims* dims, const nosa_kv* kv, const uint16_t* q,
                                       const float* score_q, const float* score_e, const int32_t* seq_lens,
                                       int32_t k_e, int32_t k_q, const uint32_t* evicted_in, uint32_t* evicted_out,
                                       int32_t* sel, int32_t sel_cap, int32_t* sel_count, const int32_t* prev,
                                       const int32_t* prev_count, int32_t* load, int32_t* load_count, int32_t* evict,
                                       int32_t* evict_count, int32_t num_splits, float sm_scale, float* o, float* m,
                                       float* l, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, kv, true)) != NOSA_OK) return st;
  if (dims->max_blocks > NOSA_SELECT_DECODE_MAX_BLOCKS) return NOSA_ERR_UNSUPPORTED;
  if (kv->kind == NOSA_TABLE_PACKED_ROPE) {
    if (!kv->q_pos || !(kv->rope_base > 1.f)) return NOSA_ERR_ARG;
    if (dims->n_q_heads / dims->n_kv_heads > 8) return NOSA_ERR_UNSUPPORTED;
  }
  if (!q || !score_q || !score_e || !seq_lens || !evicted_in || !evicted_out || !sel || !sel_count)
    return NOSA_ERR_ARG;
  if (!prev || !prev_count || !load || !load_count || !evict || !evict_count) return NOSA_ERR_ARG;
  if (!o || !m || !l) return NOSA_ERR_ARG;
  if (!aligned16(q)) return NOSA_ERR_ARG;
  if (k_e < 0 || k_q < 0 || sel_cap < 1 || sel_cap > dims->max_blocks) return NOSA_ERR_ARG;
  const int64_t k = (int64_t)k_e + k_q;
  if ((int64_t)sel_cap < (k < dims->max_blocks ? k : (int64_t)dims->max_blocks)) return NOSA_ERR_ARG;
  if (prev == sel || load == sel || evict == sel || load == evict) return NOSA_ERR_ARG;
  if (num_splits < 1 || num_splits > 256) return NOSA_ERR_ARG;
  if (num_splits > 1 && evicted_in == evicted_out) return NOSA_ERR_ARG;
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return NOSA_ERR_ARG;
  if (nosa::noalloc_layout(*dims, num_splits).total > nosa::kNoAllocScratchBytes) return NOSA_ERR_SCRATCH;
  return from_hip(nosa::launch_select_decode_noalloc(*dims, q, *kv, score_q, score_e, seq_lens, k_e, k_q,
                                                     evicted_in, evicted_out, sel, sel_cap, sel_count, prev,
                                                     prev_count, load, load_count, evict, evict_count, num_splits,
                                                     sm_scale, o, m, l, stream));
}

nosa_status nosa_host_device_pointer(const void* host_ptr, void** device_ptr) {
  if (!host_ptr || !device_ptr) return NOSA_ERR_ARG;
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<void*>(host_ptr), 0) != hipSuccess || !d) {
    (void)hipGetLastError();  // not pinned and mapped: leave no sticky error behind
    return NOSA_ERR_ARG;
  }
  *device_ptr = d;
  return NOSA_OK;
}

nosa_status nosa_retrieve(const nosa_dims* dims, const nosa_kv* host_kv, uint16_t* dev_k_pages,
                          uint16_t* dev_v_pages, float* dev_e_pages, int32_t slots, int32_t* resident,
                          int32_t* slot_owner, const int32_t* load, const int32_t* load_count, const int32_t* evict,
                          const int32_t* evict_count, int32_t cap, const int32_t* seq_lens,
                          const int32_t* seq_lens_prev, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, host_kv, true)) != NOSA_OK) return st;
  if (!dev_k_pages || !dev_v_pages || !dev_e_pages || !resident || !slot_owner || !seq_lens) return NOSA_ERR_ARG;
  if (!load || !load_count || !evict || !evict_count) return NOSA_ERR_ARG;
  if (!aligned16(dev_k_pages) || !aligned16(dev_v_pages) || !aligned16(dev_e_pages)) return NOSA_ERR_ARG;
  if (slots < 1 || slots > nosa::kMaxRetrieveSlots || cap < 1) return NOSA_ERR_ARG;
  if ((int64_t)dims->batch * dims->n_kv_heads * slots > ((int64_t)1 << 31) - 1) return NOSA_ERR_UNSUPPORTED;
  // the host pools are read through their device mapping; memory that is
  // not pinned and mapped is refused here, never dereferenced
  void *hk = nullptr, *hv = nullptr, *he = nullptr;
  if (nosa_host_device_pointer(host_kv->k_pages, &hk) != NOSA_OK) return NOSA_ERR_ARG;
  if (nosa_host_device_pointer(host_kv->v_pages, &hv) != NOSA_OK) return NOSA_ERR_ARG;
  if (nosa_host_device_pointer(host_kv->e_pages, &he) != NOSA_OK) return NOSA_ERR_ARG;
  if (!aligned16(hk) || !aligned16(hv) || !aligned16(he)) return NOSA_ERR_ARG;
  return from_hip(nosa::launch_retrieve(*dims, *host_kv, hk, hv, he, dev_k_pages, dev_v_pages, dev_e_pages, slots,
                                        resident, slot_owner, load, load_count, evict, evict_count, cap, seq_lens,
                                        seq_lens_prev, stream));
}

nosa_status nosa_retrieve_buffered(const nosa_dims* dims, const nosa_kv* host_kv, uint16_t* dev_k_pages,
                                   uint16_t* dev_v_pages, float* dev_e_pages, int32_t slots, int32_t* resident,
                                   int32_t* slot_owner, int32_t* last_use, const int32_t* sel,
                                   const int32_t* sel_count, int32_t cap, int32_t step, int32_t bucket_width,
                                   const int32_t* seq_lens, const int32_t* seq_lens_prev, int32_t* miss_count,
                                   hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if ((st = check_kv(dims, host_kv, true)) != NOSA_OK) return st;
  if (!dev_k_pages || !dev_v_pages || !dev_e_pages || !resident || !slot_owner || !last_use || !seq_lens)
    return NOSA_ERR_ARG;
  if (!sel || !sel_count) return NOSA_ERR_ARG;
  if (!aligned16(dev_k_pages) || !aligned16(dev_v_pages) || !aligned16(dev_e_pages)) return NOSA_ERR_ARG;
  if (slots < 1 || slots > nosa::kMaxRetrieveSlots || cap < 1 || cap > slots) return NOSA_ERR_ARG;
  if (step < 1 || bucket_width < 1) return NOSA_ERR_ARG;
  if ((int64_t)dims->batch * dims->n_kv_heads * slots > ((int64_t)1 << 31) - 1) return NOSA_ERR_UNSUPPORTED;
  void *hk = nullptr, *hv = nullptr, *he = nullptr;
  if (nosa_host_device_pointer(host_kv->k_pages, &hk) != NOSA_OK) return NOSA_ERR_ARG;
  if (nosa_host_device_pointer(host_kv->v_pages, &hv) != NOSA_OK) return NOSA_ERR_ARG;
  if (nosa_host_device_pointer(host_kv->e_pages, &he) != NOSA_OK) return NOSA_ERR_ARG;
  if (!aligned16(hk) || !aligned16(hv) || !aligned16(he)) return NOSA_ERR_ARG;
  return from_hip(nosa::launch_retrieve_buffered(*dims, *host_kv, hk, hv, he, dev_k_pages, dev_v_pages,
                                                 dev_e_pages, slots, resident, slot_owner, last_use, sel, sel_count,
                                                 cap, step, bucket_width, seq_lens, seq_lens_prev, miss_count,
                                                 stream));
}

nosa_status nosa_combine(const nosa_dims* dims, int32_t num_splits, const float* part_o, const float* part_m,
                         const float* part_l, float* o, float* m, float* l, hipStream_t stream) {
  nosa_status st = check_dims(dims);
  if (st != NOSA_OK) return st;
  if (num_splits < 1 || num_splits > 256 || !part_o || !part_m || !part_l || !o || !m || !l)
    return NOSA_ERR_ARG;
  return from_hip(nosa::launch_combine(*dims, num_splits, part_o, part_m, part_l, o, m, l, stream));
}

nosa_status nosa_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t n_workgroups,
                                   hipStream_t stream) {
  if (!src || !sink || !aligned16(src)) return NOSA_ERR_ARG;
  if (bytes < 16 || bytes % 16 != 0 || n_workgroups < 1 || n_workgroups > 65536) return NOSA_ERR_ARG;
  return from_hip(nosa::launch_probe_stream_read(src, bytes, sink, n_workgroups, stream));
}

nosa_status nosa_probe_page_gather(const void* k_pool, const void* v_pool, int64_t page_bytes,
                                   int64_t num_pages, const int32_t* pages, int32_t n_lists,
                                   int32_t pages_per_list, uint32_t* sink, hipStream_t stream) {
  if (!k_pool || !v_pool || !pages || !sink || !aligned16(k_pool) || !aligned16(v_pool)) return NOSA_ERR_ARG;
  if (page_bytes != 8192 && page_bytes != 16384 && page_bytes != 32768) return NOSA_ERR_ARG;
  if (num_pages < 1 || num_pages > ((int64_t)1 << 31) - 1) return NOSA_ERR_ARG;
  if (n_lists < 1 || pages_per_list < 1 || pages_per_list > 256) return NOSA_ERR_ARG;
  return from_hip(nosa::launch_probe_page_gather(k_pool, v_pool, page_bytes, num_pages, pages, n_lists,
                                                 pages_per_list, sink, stream));
}

const char* nosa_status_string(nosa_status status) {
  switch (status) {
    case NOSA_OK: return "ok";
    case NOSA_ERR_ARG: return "invalid argument";
    case NOSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case NOSA_ERR_HIP: return "HIP launch failed";
    case NOSA_ERR_SCRATCH: return "larger than the library's static scratch (NOSA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
