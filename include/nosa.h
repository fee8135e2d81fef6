/*
 * nosa.h -- C ABI of libnosa: one decode step of NOSA-style block-sparse
 * attention over a paged KV cache, on AMD Instinct MI355X (gfx950).
 *
 * The step, per (sequence b, KV head h):
 *   append      -- write this step's key/value/eviction logit, refresh the
 *                  summary of the sub-block it lands in           (support)
 *   score       -- query-aware and eviction block scores by two-stage
 *                  pooling (sub-block mean, then block max)
 *   select      -- monotone eviction set (budget k_e) + query-aware set
 *                  (budget k_q)
 *   swap_diff   -- blocks to load / drop against the previous selection
 *   decode      -- split-K flash decoding over the selected pages only
 *   combine     -- merge of the split partials into (O, rowmax, l)
 *
 * Sources (web pages, cited by title and section):
 *   [NOSA]   "NOSA: Native and Offloadable Sparse Attention" summary,
 *            gist.science 2510.13602 -- Methodology 1 (Algorithm: NOSA):
 *            dual selection, locality guarantee, block-wise two-stage
 *            pooling, ED-DMA; Methodology 2 (System: NOSI): block-sized KV
 *            layout and the set-difference kernel for block swapping.
 *   [SPIN]   "Unifying Sparse Attention with Hierarchical Memory for
 *            Scalable Long-Context LLM Serving" summary, gist.science
 *            2604.26837 -- 2.A Index/Select/Attention split over a shared
 *            page substrate; 2.B per-head physical pages; 2.C two-level
 *            page index (small GPU directory -> segments).
 *   [LAZY]   "LazyAttention" summary, gist.science 2606.04302 -- Technical
 *            implementation, 2. Decoding (query rotated only when the
 *            document changes, (block id, offset) bit-packed in one word,
 *            K and V are the only traffic); Mathematical equivalence.
 *   [NOVITA] Novita AI blog "How KV sparsity achieves 1.5x acceleration for
 *            vLLM" -- Key techniques, 2. Attention modifications (one-pass
 *            FlashAttention; rowmax and l returned with O).
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless stated otherwise, owned by the
 *     caller; the library allocates nothing and keeps no state between
 *     calls.  Calls are asynchronous on `stream` and never synchronise.
 *   - Host-side argument checks run before any launch; a failed check
 *     returns NOSA_ERR_ARG / NOSA_ERR_UNSUPPORTED and launches nothing.
 *     A failed launch returns NOSA_ERR_HIP.
 *   - Device-data contract violations (a page id outside [0, num_pages), a
 *     selected block outside [0, nb), a sequence longer than the capacity)
 *     never fault: the offending block or token is skipped and bit 0 of
 *     `nosa_kv.err_flags[0]` is set when that pointer is non-null.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Multi-index shapes are row-major; G = n_q_heads / n_kv_heads and
 *     query head j reads KV head j / G.
 *
 * Page layouts (one page = one logical block of one (b, h) pair):
 *   K page, bf16 [head_dim/8][block_size][8]: element (token t, dim d) at
 *          ((d/8) * block_size + t) * 8 + d % 8.
 *   V page, bf16 [block_size/8][head_dim][8]: element (t, d) at
 *          ((t/8) * head_dim + d) * 8 + t % 8.
 *   E page, fp32 [block_size]: eviction logit of token t.
 * Summary layouts (CS = max_blocks * nsub, nsub = block_size / sub_block):
 *   k_summary fp32 [B][Hkv][head_dim/4][CS][4]: mean key of sub-block s,
 *          dim d, at ((bh * head_dim/4 + d/4) * CS + s) * 4 + d % 4.
 *   e_summary fp32 [B][Hkv][CS]: mean eviction logit of sub-block s.
 */
#ifndef NOSA_H
#define NOSA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t nosa_status;
#define NOSA_OK               0
#define NOSA_ERR_ARG         -1  /* null pointer, bad size or shape          */
#define NOSA_ERR_UNSUPPORTED -2  /* valid but not built (head_dim, sizes)    */
#define NOSA_ERR_HIP         -3  /* a HIP launch failed                      */
#define NOSA_ERR_SCRATCH     -4  /* needs more than the static scratch       */

#define NOSA_TABLE_FLAT        0 /* table[b][h][i] -> page                   */
#define NOSA_TABLE_TWO_LEVEL   1 /* directory -> segment -> page  [SPIN 2.C] */
#define NOSA_TABLE_PACKED_ROPE 2 /* packed (page, document start) + RoPE     */

#define NOSA_PACK_PAGE_BITS 20   /* packed word: page id in bits 0..19,
                                    document start (in blocks) in bits 20..31 */

/* Sizes shared by every call.
 *   head_dim    D: 64 or 128.
 *   block_size  bs: tokens per block (= per page); 64, 128 or 256.
 *   sub_block   ss: divides bs; nsub = bs / ss is a power of two <= 64.
 *   max_blocks  logical block capacity per (b, h): 1..8192.  Sequences may
 *               hold at most max_blocks * bs tokens.
 *   n_q_heads % n_kv_heads == 0 and G = n_q_heads / n_kv_heads <= 16.    */
typedef struct nosa_dims {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t sub_block;
  int32_t max_blocks;
} nosa_dims;

/* The paged KV cache and its logical->physical page table [SPIN 2.B, 2.C].
 *   k_pages, v_pages, e_pages: num_pages pages each (layouts above).
 *   kind NOSA_TABLE_FLAT:       table int32 [B][Hkv][max_blocks].
 *   kind NOSA_TABLE_TWO_LEVEL:  key = ((b*Hkv + h) << blocks_log2) | i;
 *        seg = directory[key >> seg_log2] (int32 [dir_entries], -1 = none);
 *        page = segments[(seg << seg_log2) | (key & (2^seg_log2 - 1))]
 *        (int32 [num_segments << seg_log2]).  Requires
 *        max_blocks <= 2^blocks_log2, seg_log2 <= blocks_log2 and
 *        dir_entries >= (B*Hkv << blocks_log2) >> seg_log2.
 *   kind NOSA_TABLE_PACKED_ROPE [LAZY 2. Decoding]: packed uint32
 *        [B][Hkv][max_blocks]; page = word & 0xFFFFF, document start
 *        position = (word >> 20) * block_size.  q_pos int32 [B] is the
 *        query position n; stored keys carry the rotation of their position
 *        inside their document, and decode scores block tokens with the
 *        query rotated by n - document start (rotate-half RoPE,
 *        theta_i = rope_base^(-2i/D)).  Only nosa_sparse_decode applies the
 *        rotation; the other calls use the packed word for the page only.
 *   err_flags: optional int32 [1]; bit 0 is set on a device-data contract
 *        violation (see above).  Never cleared by the library.            */
typedef struct nosa_kv {
  uint16_t* k_pages;
  uint16_t* v_pages;
  float* e_pages;
  int64_t num_pages;
  int32_t kind;
  int32_t dir_entries;
  const int32_t* table;
  const int32_t* directory;
  const int32_t* segments;
  int64_t num_segments;
  int32_t seg_log2;
  int32_t blocks_log2;
  const uint32_t* packed;
  const int32_t* q_pos;
  float rope_base;
  int32_t* err_flags;
} nosa_kv;

/* Index op [SPIN 2.A]: copy the first seq_lens[b] tokens of every (b, h)
 * from contiguous sources into their pages.
 *   k_src, v_src: bf16 [B][Hkv][src_tokens][D];  e_src: fp32 [B][Hkv][src_tokens].
 *   seq_lens int32 [B], each <= min(src_tokens, max_blocks * bs).
 * Page slots past seq_lens[b] are left as they are, except that unused
 * token slots of a partially filled V group of 8 are written with zeros.   */
nosa_status nosa_prefill_pages(const nosa_dims* dims, const nosa_kv* kv,
                               const uint16_t* k_src, const uint16_t* v_src, const float* e_src,
                               int32_t src_tokens, const int32_t* seq_lens, hipStream_t stream);

/* Index op, pooling inputs [NOSA block-wise implementation; NOSI fused
 * pooling]: the fp32 mean key and mean eviction logit of every non-empty
 * sub-block of every (b, h), over its present tokens (sum in float64 in
 * token order, one rounding to fp32).  Entries of empty sub-blocks are not
 * written.  Layouts above.                                                  */
nosa_status nosa_build_summaries(const nosa_dims* dims, const nosa_kv* kv, const int32_t* seq_lens,
                                 float* k_summary, float* e_summary, hipStream_t stream);

/* Decode-step append: token T = seq_lens[b] of every (b, h) gets
 *   k_new, v_new: bf16 [B][Hkv][D];  e_new: fp32 [B][Hkv];
 * the summary of the sub-block holding it is recomputed exactly as
 * nosa_build_summaries would, and seq_lens[b] becomes T + 1 (in place).
 * The page of the block holding token T must exist in the table.          */
nosa_status nosa_append(const nosa_dims* dims, const nosa_kv* kv,
                        const uint16_t* k_new, const uint16_t* v_new, const float* e_new,
                        int32_t* seq_lens, float* k_summary, float* e_summary, hipStream_t stream);

/* Select, scoring [NOSA dual selection, block-wise implementation, ED-DMA]:
 * for block i < nb = ceil(T / bs), T = seq_lens[b],
 *   score_q[b][h][i] = max over non-empty sub-blocks j of
 *                      (qbar . kbar_ij) / sqrt(D),  qbar = mean of the G
 *                      query heads of KV head h (the group-mean per-token
 *                      score, mean-pooled, by linearity), float64
 *                      accumulation, rounded once to fp32;
 *   score_e[b][h][i] = max over non-empty sub-blocks of the mean eviction
 *                      logit (raw logits, no exponent).
 *   q: bf16 [B][Hq][D].  score_q, score_e: fp32 [B][Hkv][max_blocks];
 * entries i >= nb are not written.  The query is taken as stored keys are:
 * for a cache with deferred RoPE (packed table) score through
 * nosa_append_score, which takes the descriptor and rotates the query.    */
nosa_status nosa_score_blocks(const nosa_dims* dims, const uint16_t* q,
                              const float* k_summary, const float* e_summary, const int32_t* seq_lens,
                              float* score_q, float* score_e, hipStream_t stream);

/* Select, dual selection [NOSA dual selection, locality guarantee]:
 *   candidates C = { i < nb : evicted bit i clear };
 *   Gamma_e = the min(k_e, |C|) best of C by (score_e desc, i asc); every
 *             other candidate gets its evicted bit set (never cleared);
 *   Gamma_q = the min(k_q, nb - |Gamma_e|) best of the blocks not in
 *             Gamma_e by (score_q desc, i asc);
 *   sel[b][h][0 .. sel_count) = Gamma_e U Gamma_q, ascending.
 * After the call Gamma_e = { i < nb : evicted bit i clear }.
 *   evicted: uint32 [B][Hkv][ceil(max_blocks / 32)], bit i of word i/32;
 *            in/out, all zero before the first step.
 *   sel: int32 [B][Hkv][sel_cap], sel_cap >= min(k_e + k_q, max_blocks);
 *   sel_count: int32 [B][Hkv].  k_e, k_q >= 0.                             */
nosa_status nosa_select(const nosa_dims* dims, const float* score_q, const float* score_e,
                        const int32_t* seq_lens, int32_t k_e, int32_t k_q, uint32_t* evicted,
                        int32_t* sel, int32_t sel_cap, int32_t* sel_count, hipStream_t stream);

/* nosa_append_score from the token's fused projection row [NOSA, NOSI
 * kernel fusion: the eviction head, the QKV split and pooling in one
 * kernel]:
 *   qkv bf16 [B][(Hq + 2 Hkv) D]: per sequence the new token's row
 *     [q heads | k heads | v heads];
 *   w_evict fp32 [Hkv][D]: the eviction head, e = w_h . v (float64 sum,
 *     one rounding to fp32), no exponent [NOSA, ED-DMA];
 *   q_out bf16 [B][Hq][D]: receives the query part (the decode's q).
 * The token's k, v and e are appended and the blocks scored with the row's
 * query exactly as nosa_append_score does with k_new, v_new, e_new and q
 * (seq_lens_in / seq_lens_out, k_summary .. score_e as there).  Flat and
 * two-level tables (NOSA_ERR_UNSUPPORTED for the packed RoPE kind).       */
nosa_status nosa_append_score_qkv(const nosa_dims* dims, const nosa_kv* kv, const uint16_t* qkv,
                                  const float* w_evict, const int32_t* seq_lens_in, int32_t* seq_lens_out,
                                  float* k_summary, float* e_summary, uint16_t* q_out, float* score_q,
                                  float* score_e, hipStream_t stream);

/* nosa_select and nosa_swap_diff in one launch: the selection is made as
 * by nosa_select, then load / evict are formed against prev exactly as
 * nosa_swap_diff(prev, sel) would, from the selection still in registers
 * (saves a launch and a round trip on the decode step).  prev, load and
 * evict are int32 [B][Hkv][sel_cap] with counts [B][Hkv]; here
 * sel_cap <= max_blocks, and sel, prev, load, evict must be distinct.    */
nosa_status nosa_select_swap(const nosa_dims* dims, const float* score_q, const float* score_e,
                             const int32_t* seq_lens, int32_t k_e, int32_t k_q, uint32_t* evicted,
                             int32_t* sel, int32_t sel_cap, int32_t* sel_count,
                             const int32_t* prev, const int32_t* prev_count,
                             int32_t* load, int32_t* load_count, int32_t* evict, int32_t* evict_count,
                             hipStream_t stream);

/* nosa_append and nosa_score_blocks in one launch [NOSA, NOSI: pooling
 * fused into the index-side kernel].  Results are bit-identical to the two
 * calls in sequence, except for where the new lengths go:
 *   k_new, v_new, e_new: as nosa_append, or all NULL for no append;
 *   seq_lens_in int32 [B]: lengths before the append (read only);
 *   seq_lens_out int32 [B]: written with the lengths after the append
 *     (seq_lens_in[b] + 1, or unchanged where the append is out of range,
 *     which also sets the error flag); required with an append and must
 *     differ from seq_lens_in; ignored (may be NULL) without one;
 *   k_summary, e_summary, q, score_q, score_e: as nosa_append /
 *     nosa_score_blocks.
 * Scoring uses the lengths after the append.
 * With a NOSA_TABLE_PACKED_ROPE descriptor (scoring only: no append, and
 * 4 <= block_size / sub_block <= 16, else NOSA_ERR_UNSUPPORTED; q_pos and
 * rope_base required) the stored keys carry their in-document rotation
 * [LAZY, 2. Decoding], and score_q of a block in the document starting at
 * position st is taken with the group's mean query turned by q_pos[b] - st:
 *   score_q[i] = max_j Rot(q_pos - st) qbar . kbar_ij / sqrt(D),
 * which equals the sub-block mean of Rot(q_pos) q . Rot(st) k_stored over
 * the group; score_e is as without RoPE.                                  */
nosa_status nosa_append_score(const nosa_dims* dims, const nosa_kv* kv,
                              const uint16_t* k_new, const uint16_t* v_new, const float* e_new,
                              const int32_t* seq_lens_in, int32_t* seq_lens_out,
                              float* k_summary, float* e_summary, const uint16_t* q,
                              float* score_q, float* score_e, hipStream_t stream);

/* Block-swap set differences [NOSA, NOSI set-difference kernel]:
 *   load  = cur  minus prev (in cur's order),
 *   evict = prev minus cur  (in prev's order),
 * per (b, h), over lists int32 [B][Hkv][cap] with counts int32 [B][Hkv].
 * Entries must lie in [0, max_blocks) and a list holds no duplicates;
 * entries outside that range are skipped.  Outputs may not alias inputs. */
nosa_status nosa_swap_diff(const nosa_dims* dims, int32_t cap,
                           const int32_t* prev, const int32_t* prev_count,
                           const int32_t* cur, const int32_t* cur_count,
                           int32_t* load, int32_t* load_count,
                           int32_t* evict, int32_t* evict_count, hipStream_t stream);

/* Attention, split-K over the selected pages [NOVITA one-pass FlashAttention;
 * LAZY decoding for NOSA_TABLE_PACKED_ROPE].  The selected list of (b, h)
 * is cut into num_splits contiguous chunks of ceil(n / num_splits) blocks;
 * for chunk p and query head j of the group,
 *   s = sm_scale * q_j . k over the present tokens of the chunk's blocks,
 *   part_m = max s, part_l = sum exp(s - part_m),
 *   part_o = sum exp(s - part_m) v / part_l;
 * an empty chunk gives part_m = -inf, part_l = 0, part_o = 0.
 *   q: bf16 [B][Hq][D];  sel: int32 [B][Hkv][sel_cap];  sel_count [B][Hkv];
 *   part_o fp32 [B][Hq][num_splits][D];  part_m, part_l fp32 [B][Hq][num_splits].
 * 1 <= num_splits <= 256.                                                  */
nosa_status nosa_sparse_decode(const nosa_dims* dims, const uint16_t* q, const nosa_kv* kv,
                               const int32_t* sel, const int32_t* sel_count, int32_t sel_cap,
                               const int32_t* seq_lens, int32_t num_splits, float sm_scale,
                               float* part_o, float* part_m, float* part_l, hipStream_t stream);

/* nosa_sparse_decode and nosa_combine in one launch: the decode writes its
 * split partials as above, and the last workgroup of each (b, h) to finish
 * (counted with a device-scope atomic in counters[b*Hkv + h]) merges them
 * into o, m, l exactly as nosa_combine defines.
 *   counters: int32 [B][Hkv], all zero before the first call; every call
 *   leaves them zero.  Calls that overlap on the same counters race.      */
nosa_status nosa_sparse_decode_combine(const nosa_dims* dims, const uint16_t* q, const nosa_kv* kv,
                                       const int32_t* sel, const int32_t* sel_count, int32_t sel_cap,
                                       const int32_t* seq_lens, int32_t num_splits, float sm_scale,
                                       float* part_o, float* part_m, float* part_l, int32_t* counters,
                                       float* o, float* m, float* l, hipStream_t stream);

/* nosa_sparse_decode_combine with the softmax score step [NOVITA, 2.
 * Attention modifications: with the returned row max and l, p =
 * exp(q.k - rowmax) / l is each key's softmax score, summed row-wise into a
 * sparsification score].  Besides o, m, l (bit-identical to
 * nosa_sparse_decode_combine):
 *   mass fp32 [B][Hq][sel_cap]: mass[b][j][s] = the sum of query head j's
 *     probabilities exp(s_t - m) / l over the present tokens of block
 *     sel[b][h][s] (h = j / G), so each head's row sums to 1 over the
 *     selection; entries at or past sel_count and blocks the table cannot
 *     resolve receive 0;
 *   tile_stats fp32 [B][Hkv][sel_cap * block_size / 64][G][2]: workspace
 *     (per 64-token tile and head: the sum of its probabilities and the
 *     running max they are relative to), written and read by the call.
 * The keys are read once: the mass comes from statistics of the decode's
 * own tiles.  Flat and two-level tables (NOSA_ERR_UNSUPPORTED for the
 * packed RoPE kind).                                                      */
nosa_status nosa_sparse_decode_mass(const nosa_dims* dims, const uint16_t* q, const nosa_kv* kv,
                                    const int32_t* sel, const int32_t* sel_count, int32_t sel_cap,
                                    const int32_t* seq_lens, int32_t num_splits, float sm_scale,
                                    float* part_o, float* part_m, float* part_l, int32_t* counters,
                                    float* o, float* m, float* l, float* tile_stats, float* mass,
                                    hipStream_t stream);

/* nosa_sparse_decode_combine with ALiBi position biases [LAZY,
 * generalisation: the deferred treatment of positions carries over to
 * relative schemes such as ALiBi; keys are stored without positions and
 * the bias is applied at attention time]:
 *   s = sm_scale * q_j . k_t - alibi_slopes[j] * (n - t)
 * for query head j, key position t (its logical token index) and query
 * position n = seq_lens[b] - 1 (the newest token); everything else as
 * nosa_sparse_decode_combine.
 *   alibi_slopes fp32 [Hq] (device), e.g. 2^(-8 (j + 1) / Hq).
 * Flat and two-level tables (NOSA_ERR_UNSUPPORTED for the packed RoPE
 * kind).                                                                  */
nosa_status nosa_sparse_decode_alibi(const nosa_dims* dims, const uint16_t* q, const nosa_kv* kv,
                                     const int32_t* sel, const int32_t* sel_count, int32_t sel_cap,
                                     const int32_t* seq_lens, int32_t num_splits, float sm_scale,
                                     const float* alibi_slopes, float* part_o, float* part_m, float* part_l,
                                     int32_t* counters, float* o, float* m, float* l, hipStream_t stream);

/* nosa_select_swap and nosa_sparse_decode_combine in one launch [SPIN 2.A:
 * Select and Attention kept as stages of one launch].  Every workgroup of
 * a (b, h) pair makes the pair's selection from score_q / score_e into
 * on-chip memory, exactly as nosa_select_swap, and decodes its split of it;
 * the workgroup of split 0 also writes the selection, the new eviction
 * bitmap and the swap lists.  The selection, bitmap and swap lists are
 * bit-identical to nosa_select_swap's, except that the bitmap is read from
 * evicted_in and written to evicted_out; o, m, l are the same attention as
 * nosa_sparse_decode_combine's over that selection, up to the order in
 * which tiles are accumulated (m bit-identical).  How the splits divide
 * the selection:
 *   - when the eviction part keeps every block it has not dropped (all
 *     steps but those where a new block competes [NOSA summary,
 *     Methodology 1, locality guarantee]), split p takes the p-th of P
 *     equal shares, in whole blocks, of the eviction part and of the query
 *     part: eviction blocks [p n_e / P, (p+1) n_e / P) of its ascending
 *     list and query blocks [p n_q / P, (p+1) n_q / P) of its own, where
 *     n_e is the number of blocks below ceil(seq_len / block_size) clear in
 *     evicted_in and n_q = min(k_q, nb - n_e) (integer division);
 *   - otherwise split p takes the p-th contiguous chunk of the ascending
 *     list, as nosa_sparse_decode_combine;
 *   part_o / part_m / part_l then hold those splits' partials.
 *   evicted_in, evicted_out: uint32 [B][Hkv][ceil(max_blocks / 32)]; the
 *     same buffer is allowed only with num_splits == 1;
 *   score_q, score_e, seq_lens, k_e, k_q, sel .. evict_count: as
 *     nosa_select_swap (sel_cap <= max_blocks);
 *   q, num_splits, sm_scale, part_* , counters, o, m, l: as
 *     nosa_sparse_decode_combine (packed RoPE kind: q_pos and rope_base
 *     in kv, and at most 8 query heads per KV head).
 * Supported with max_blocks <= NOSA_SELECT_DECODE_MAX_BLOCKS
 * (NOSA_ERR_UNSUPPORTED otherwise: make the two calls).                   */
#define NOSA_SELECT_DECODE_MAX_BLOCKS 2304
nosa_status nosa_select_decode(const nosa_dims* dims, const nosa_kv* kv, const uint16_t* q,
                               const float* score_q, const float* score_e, const int32_t* seq_lens,
                               int32_t k_e, int32_t k_q, const uint32_t* evicted_in, uint32_t* evicted_out,
                               int32_t* sel, int32_t sel_cap, int32_t* sel_count,
                               const int32_t* prev, const int32_t* prev_count,
                               int32_t* load, int32_t* load_count, int32_t* evict, int32_t* evict_count,
                               int32_t num_splits, float sm_scale, float* part_o, float* part_m, float* part_l,
                               int32_t* counters, float* o, float* m, float* l, hipStream_t stream);

/* nosa_select_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same launch and results, bit for bit, as
 * nosa_select_decode, but the split partials and the arrival counters of the
 * fused combine live in a fixed device array of the library
 * (NOSA_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends) instead
 * of caller buffers; the caller passes every input and output, and the call
 * allocates nothing.
 *   Arguments: as nosa_select_decode without part_o, part_m, part_l and
 *     counters.
 *   Size limit: 256 KiB of counters plus the partials, 4 B * B * Hq * P * (D
 *     + 2) rounded up, must fit NOSA_NOALLOC_SCRATCH_BYTES (16 MiB: e.g. B =
 *     32, Hq = 32, D = 128 up to P = 31); larger calls return
 *     NOSA_ERR_SCRATCH and launch nothing.
 *   Set-up: the first call on a device looks up that device's copy of the
 *     array and clears its counters with a small kernel on `stream`; make
 *     that first call outside graph capture.
 *   Sharing: every call on a GPU uses that GPU's array, which keeps the
 *     last call's contents; each call leaves the counters zero.  Calls that
 *     overlap on one GPU (concurrent streams or threads) race: serialise
 *     them.                                                               */
#define NOSA_NOALLOC_SCRATCH_BYTES (16ll << 20)
nosa_status nosa_select_decode_noalloc(const nosa_dims* dims, const nosa_kv* kv, const uint16_t* q,
                                       const float* score_q, const float* score_e, const int32_t* seq_lens,
                                       int32_t k_e, int32_t k_q, const uint32_t* evicted_in, uint32_t* evicted_out,
                                       int32_t* sel, int32_t sel_cap, int32_t* sel_count,
                                       const int32_t* prev, const int32_t* prev_count,
                                       int32_t* load, int32_t* load_count, int32_t* evict, int32_t* evict_count,
                                       int32_t num_splits, float sm_scale, float* o, float* m, float* l,
                                       hipStream_t stream);

/* Retrieve: the host tier [NOSA, Methodology 2 (NOSI): block-sized KV
 * units, set differences drive block swapping, a host-to-device transfer
 * kernel over unified virtual addressing; SPIN 2.A: Offload / Retrieve as
 * system-managed operations; 2.B: per-head pages].
 *   host_kv: the whole paged cache in pinned host memory: k_pages, v_pages,
 *     e_pages are HOST pointers (allocated pinned and mapped, e.g. by
 *     hipHostMalloc); its table / directory / segments / packed words map
 *     logical blocks to host pages as in nosa_kv (device pointers).
 *   dev_k_pages, dev_v_pages, dev_e_pages: the resident pools in HBM,
 *     B * Hkv * slots pages, same page layouts; device page bh * slots + s
 *     is slot s of pair bh (bh = b * Hkv + h).
 *   resident int32 [B][Hkv][max_blocks]: device page of each resident
 *     logical block, -1 elsewhere (the flat table a decode over the
 *     resident pools takes); slot_owner int32 [B][Hkv][slots]: logical
 *     block in each slot, -1 for a free slot.  Both all -1 before the first
 *     call; the library keeps them consistent.
 *   load / evict (+ counts), cap: the swap lists of this step (as produced
 *     by nosa_swap_diff or nosa_select_swap).
 *   seq_lens int32 [B]: lengths after this step's append.
 *   seq_lens_prev int32 [B] or null: the lengths at the previous call; the
 *     tokens [seq_lens_prev[b], seq_lens[b]) were appended into the host
 *     pools since then.
 * Per pair: every evicted block frees its slot; the j-th loaded block takes
 * the j-th free slot in ascending slot order and its K, V and E pages are
 * copied from host memory into it (zero-copy reads by the kernel).  Every
 * other resident block holding appended tokens gets those tokens copied
 * (K: their D/8 16-byte units; V: the 8-token rows that hold them; E: the
 * 4-token units that hold them); with seq_lens_prev null the resident
 * block holding the last token is copied whole instead.  More loads than
 * free slots set the error flag and the excess blocks stay out.
 * 1 <= slots <= 1024.                                                     */
nosa_status nosa_retrieve(const nosa_dims* dims, const nosa_kv* host_kv,
                          uint16_t* dev_k_pages, uint16_t* dev_v_pages, float* dev_e_pages, int32_t slots,
                          int32_t* resident, int32_t* slot_owner,
                          const int32_t* load, const int32_t* load_count,
                          const int32_t* evict, const int32_t* evict_count, int32_t cap,
                          const int32_t* seq_lens, const int32_t* seq_lens_prev, hipStream_t stream);

/* Retrieve with a locality-aware buffer [SPIN 2.B: the GPU buffer of a
 * request holds the pages the current step needs plus buffered pages kept
 * for temporal locality; buffered pages are evicted by a bucketed LRU over
 * recency timestamps (e.g. 64 buckets), decided in parallel on the GPU
 * without a global sort].
 *   host_kv, dev_*_pages, resident, slot_owner: as nosa_retrieve, with
 *     cap <= slots <= 1024 (slots beyond cap are the buffer).
 *   last_use int32 [B][Hkv][slots]: the step at which each slot's block was
 *     last selected (ignored for free slots); kept by the library.
 *   sel, sel_count, cap: this step's selection (ascending block ids).
 *   step: this step's number, >= 1, larger than every earlier step.
 *   bucket_width: steps per recency bucket (>= 1).
 *   miss_count int32 [B][Hkv] or null: pages loaded per pair.
 * Per pair: selected blocks already resident are hits (timestamp := step);
 * the others are misses.  When the free slots are fewer than the misses,
 * buffered pages (resident, not selected) are dropped, oldest first by
 * bucket = min((step - last_use - 1) / bucket_width, 63), lowest slot first
 * inside the bucket where dropping stops.  The j-th miss (selection order)
 * takes the j-th free slot in ascending order (timestamp := step) and its
 * K, V and E pages are copied from host memory; appended tokens reach the
 * resident pages as in nosa_retrieve (seq_lens_prev as there).  The swap
 * lists are not needed.                                                   */
nosa_status nosa_retrieve_buffered(const nosa_dims* dims, const nosa_kv* host_kv,
                                   uint16_t* dev_k_pages, uint16_t* dev_v_pages, float* dev_e_pages,
                                   int32_t slots, int32_t* resident, int32_t* slot_owner, int32_t* last_use,
                                   const int32_t* sel, const int32_t* sel_count, int32_t cap, int32_t step,
                                   int32_t bucket_width, const int32_t* seq_lens,
                                   const int32_t* seq_lens_prev, int32_t* miss_count, hipStream_t stream);

/* The device address of pinned, mapped host memory (to pass host pools to
 * the calls that read or write pages through a kernel, e.g. an append into
 * the host tier).  NOSA_ERR_ARG for memory that is not pinned and mapped. */
nosa_status nosa_host_device_pointer(const void* host_ptr, void** device_ptr);

/* Prefill over reused documents with deferred RoPE [LAZY, 1. Prefilling:
 * a single relative rotation from the offset between the queries and the
 * cached document instead of re-encoding the keys; Mathematical
 * equivalence].  The prompt (n_prompt tokens, query m at position
 * n = q_pos0[b] + m) attends causally over the context: the keys at
 * positions t <= n, t < seq_lens[b], with the prompt's own keys already in
 * the cache as its last document.  Stored keys carry their in-document
 * rotation (as for nosa_sparse_decode with NOSA_TABLE_PACKED_ROPE), so
 *   s = sm_scale * Rot(n - st) q_j . k_stored,  st = the document start
 * of the key's block (from the packed word); every block up to the last
 * position is read (no selection).
 *   q bf16 [B][n_prompt][Hq][D] (unrotated);  q_pos0, seq_lens int32 [B];
 *   o fp32 [B][n_prompt][Hq][D];  m, l fp32 [B][n_prompt][Hq] (natural-log
 *   units, as nosa_combine).
 * NOSA_TABLE_PACKED_ROPE descriptors only (rope_base required); block_size
 * a multiple of 64.                                                       */
nosa_status nosa_prefill_attention(const nosa_dims* dims, const nosa_kv* kv, const uint16_t* q,
                                   int32_t n_prompt, const int32_t* q_pos0, const int32_t* seq_lens,
                                   float sm_scale, float* o, float* m, float* l, hipStream_t stream);

/* Attention, combine [NOVITA: return rowmax and l with O]:
 *   m = max_p part_m (over p with part_l > 0), l = sum_p part_l e^(part_m - m),
 *   O = sum_p part_l e^(part_m - m) part_o / l;  all empty: O = 0, m = -inf, l = 0.
 *   o fp32 [B][Hq][D];  m, l fp32 [B][Hq] (natural-log units of s).        */
nosa_status nosa_combine(const nosa_dims* dims, int32_t num_splits,
                         const float* part_o, const float* part_m, const float* part_l,
                         float* o, float* m, float* l, hipStream_t stream);

/* Bandwidth probes (measurement tools, not part of the step): the HBM read
 * rate this GPU gives the step's two access patterns with no arithmetic on
 * the data, to set the step's kernels against.  Each workgroup writes the
 * xor of every 32-bit word it read to sink[workgroup] (so the xor of the
 * sink equals the xor of the bytes read, a check that all of them were).
 *
 * nosa_probe_stream_read: `bytes` (a multiple of 16, src 16-byte aligned)
 *   read once, contiguously, with 16-byte non-temporal loads (the pattern
 *   of the block-summary stream); n_workgroups in [1, 65536] workgroups of
 *   256 threads; sink uint32 [n_workgroups].
 * nosa_probe_page_gather: the K page and the V page of every page id in
 *   pages int32 [n_lists][pages_per_list] read whole from k_pool / v_pool
 *   (page_bytes 8192, 16384 or 32768; pages [0, num_pages); ids outside are
 *   skipped): the decode's selected-page gather, one workgroup of four waves
 *   per list (a (b, h) pair), wave w taking pages w, w + 4, ..., one K page
 *   and one V page in flight per wave.  pages_per_list in [1, 256];
 *   sink uint32 [n_lists].
 * NOSA_ERR_ARG on null or misaligned pointers and sizes out of range.     */
nosa_status nosa_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t n_workgroups,
                                   hipStream_t stream);
nosa_status nosa_probe_page_gather(const void* k_pool, const void* v_pool, int64_t page_bytes,
                                   int64_t num_pages, const int32_t* pages, int32_t n_lists,
                                   int32_t pages_per_list, uint32_t* sink, hipStream_t stream);

/* Static description of a status code (never null). Host only.           */
const char* nosa_status_string(nosa_status status);

#ifdef __cplusplus
}
#endif

#endif /* NOSA_H */
