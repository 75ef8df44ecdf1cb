/*
 * libmla -- Multi-head Latent Attention (MLA) decode in its weight-absorbed form,
 * for AMD Instinct MI355X (gfx950).
 *
 * One decode step of one attention layer, for a batch of sequences whose keys
 * and values are kept only as the cached joint latent c^KV (d_c values) and the
 * head-shared, already position-encoded RoPE key k^R (d_h^R values) per token:
 *
 *   mla_absorb_q        q~_i = (W^UK_i)^T q^C_i, and RoPE_p(q^R_i)           (per head i)
 *   mla_plan_splits     cut every sequence's pages into work items (host)
 *   mla_plan_splits_ordered  the same, sized for longest-first dispatch, and the order
 *   mla_decode_splitkv  per work item: scores against [c^KV | k^R], online
 *                       softmax, latent-space weighted sum, partial LSE
 *   mla_decode_splitkv_ordered  the same, items started in a given order
 *   mla_combine         log-sum-exp merge of the work items of a sequence
 *   mla_decode_merged   the two above in one launch
 *   mla_decode_splitkv_multi, mla_combine_multi
 *                       the same for q_len query tokens per sequence (causal)
 *   mla_prefill_naive   q_len query tokens per sequence through the materialised
 *                       per-head K/V path (for long chunks, where it costs less)
 *   mla_append_kv       write the decoded token's [c^KV | RoPE(k^R)] row into the cache
 *   mla_append_kv_noalloc  the same without a workspace argument (static scratch)
 *   mla_out_proj        o_i = W^UV_i o~_i                                    (per head i)
 *   mla_combine_out_proj  mla_combine and mla_out_proj in one launch
 *
 * Pages describing the method (titles as published):
 *   "DeepSeek V2 技术解析：多头潜在注意力（MLA）与混合专家模型（MoE）的创新实践",
 *       part 2, sections 2.2.1.1 (joint KV compression, absorption remark) and
 *       2.2.2 (decoupled RoPE, what is cached);
 *   "DeepSeek-V2/V3：大模型的两张账，为什么 MLA 与 MoE 要一起看", section
 *       "第一张账" (scores read the cached latent through the transformed query,
 *       aggregation happens in latent space) and the RoPE section (content and
 *       position channels, per-head q^R, one shared k^R, concatenated inner product).
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * Memory: every pointer argument, unless its name ends in _host, is a device
 *   pointer on the current HIP device.  The caller allocates and owns all
 *   buffers; the library allocates nothing, frees nothing and keeps no pointer
 *   after a call returns.  Calls keep no state between them.  The one
 *   exception is mla_append_kv_noalloc, whose scratch is a static device
 *   buffer of the library (see there).
 * Streams: `stream` is a hipStream_t (NULL = the default stream).  Kernels are
 *   enqueued on it and the call returns without synchronising.
 * Errors: arguments are checked on the host before any HIP call; a failed check
 *   returns a negative status and enqueues nothing.  A failed launch returns
 *   MLA_ERR_HIP.  Device data is not checked: a block-table entry outside
 *   [0, num_pages) or a length outside [1, max_pages_per_seq * page_size] is
 *   undefined behaviour (mla_check_paging looks for both, for debugging).  No
 *   C++ exception crosses this interface.
 * Layouts (row-major, innermost last; "dtype" is mla_dims.dtype):
 *   q_nope      [batch][n_heads][d_head]                 dtype
 *   q_pe        [batch][n_heads][d_rope]                 dtype (not yet encoded)
 *   positions   [batch]                                  int32 (RoPE position of the query)
 *   w_uk, w_uv  [n_heads * d_head][d_latent]             dtype; head i owns rows
 *               i*d_head .. i*d_head + d_head - 1 (k^C = W^UK c^KV, v^C = W^UV c^KV)
 *   q_abs       [batch][n_heads][d_latent + d_rope]      dtype: [q~_i | RoPE_p(q^R_i)]
 *   kv_cache    [num_pages][page_size][d_latent + d_rope] dtype: one row per token,
 *               [c^KV_j | k^R_j], k^R_j already encoded at its own position
 *   block_table [batch][max_pages_per_seq]               int32: token j of sequence b
 *               is row (j % page_size) of page block_table[b][j / page_size]
 *   seq_lens    [batch]                                  int32: tokens 0..seq_lens[b]-1
 *               are attended (seq_lens[b] >= 1)
 *   items       [num_items][4]                           int32: (b, split, page_begin, page_end)
 *   split_offsets [batch + 1]                            int32: items of sequence b are
 *               split_offsets[b] .. split_offsets[b+1]-1, in token order; every
 *               sequence has at least one item (as mla_plan_splits makes them)
 *   o_part      [num_items][n_heads][d_latent]           float32
 *   lse_part    [num_items][n_heads]                     float32 (natural log)
 *   o_latent    [batch][n_heads][d_latent]               float32: o~_i
 *   lse         [batch][n_heads]                         float32 (natural log)
 *   out         [batch][n_heads][d_head]                 float32: o_i
 * Alignment: device pointers of dtype or float32 arrays must be 16-byte aligned.
 * Numerics: bf16 operands with float32 accumulation; softmax in float32; RoPE
 *   angles p * theta_k in float64 and the rotation in float32.  The sine/cosine
 *   are float64 except in the gfx950 fast absorb, which reduces the float64
 *   angle to [-pi, pi] in float64 and takes them in float32 (within about one
 *   float32 ulp of the float64 values).
 *   The fast decode kernels weigh tokens against a per-head reference that
 *   starts at the work item's first-slice score maximum and moves up to a later
 *   slice's maximum when that passes it by more than 2^8 (the accumulators are
 *   rescaled then); MLA_DECODE_MAX_JUMP (log2 units, in (0, 30]) sets that
 *   threshold.  With up to 64 heads per workgroup (every head count but 16)
 *   the two halves of a slice's tokens are scored by different waves, which agree on moves once per window of 8 slices (256
 *   tokens), from that window's maxima, so within a window the weights can
 *   pass the reference by the window's rise; if one passes 2^64 the item is
 *   recomputed against exact maxima (read the count with
 *   mla_decode_exact_pass_count; MLA_DECODE_SAFE_JUMP, in (0, 100], lowers
 *   that bound).  The result is the same softmax either way.
 *
 * Supported shapes: the gfx950 fast path needs dtype MLA_BF16, d_latent 512,
 * d_rope 64, d_head 128, page_size 64 and n_heads a multiple of 16 (the
 * decode gives a work item one workgroup at 16 heads, else ceil(n_heads / 64)
 * workgroups of up to 64 heads); any other shape
 * with d_latent <= 1024, d_rope even and <= 128, d_head <= 256, page_size in
 * [1, 1024] and n_heads <= 1024 runs on straightforward kernels; larger ones
 * return MLA_ERR_UNSUPPORTED.
 */
#ifndef MLA_H
#define MLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_VERSION 100 /* major * 100 + minor */

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, L_b < 1 */
  MLA_ERR_UNSUPPORTED = -2, /* shape or dtype this library does not handle */
  MLA_ERR_WORKSPACE = -3,   /* caller-provided capacity too small */
  MLA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} mla_status;

typedef enum { MLA_BF16 = 0, MLA_F32 = 1 } mla_dtype;

typedef struct {
  int32_t n_heads;     /* n_h */
  int32_t d_head;      /* d_h: width of q^C and of the output o_i */
  int32_t d_latent;    /* d_c: width of the cached latent c^KV */
  int32_t d_rope;      /* d_h^R: width of q^R and of the shared key k^R (even) */
  int32_t page_size;   /* tokens per cache page */
  float softmax_scale; /* multiplies q . k; the usual value is 1/sqrt(d_head + d_rope) */
  double rope_base;    /* theta_k = rope_base^(-2k/d_rope), pairs (2k, 2k+1) */
  mla_dtype dtype;     /* storage type of q_nope, q_pe, q_abs, kv_cache, w_uk, w_uv */
} mla_dims;

/* Absorb W^UK into the query and encode the RoPE part.
 * Page "DeepSeek V2 技术解析" 2.2.1.1 (W^UK absorbed on the query side) and 2.2.2
 * (decoupled per-head q^R carries the position; R_m rotation).
 * For every (b, i): q_abs[b][i][0:d_latent] = (W^UK_i)^T q_nope[b][i] rounded to dtype,
 * q_abs[b][i][d_latent:] = RoPE_{positions[b]}(q_pe[b][i]) rounded to dtype, where RoPE
 * rotates the pair (x_2k, x_2k+1) by positions[b] * rope_base^(-2k/d_rope) radians:
 * (x_2k cos - x_2k+1 sin, x_2k sin + x_2k+1 cos).
 * Errors: MLA_ERR_INVALID_ARG for null pointers, batch < 1 or misalignment. */
mla_status mla_absorb_q(const mla_dims* dims, int32_t batch, const void* q_nope, const void* q_pe,
                        const int32_t* positions, const void* w_uk, void* q_abs, void* stream);

/* Plan the split-KV work items (host only, no HIP call, deterministic).
 * Each sequence's pages 0 .. ceil(L_b / page_size)-1 are cut into contiguous,
 * non-empty page ranges; every page of every sequence lands in exactly one item.
 * The item size is chosen so that about `num_slots` workgroups (CUs times
 * workgroups resident per CU) stay busy with even loads; on the gfx950 fast
 * path each item is decoded by one workgroup at 16 heads and otherwise by
 * ceil(n_heads / 64) (two at 128 heads, one per half of the heads), so about
 * num_slots divided by that many items are made.
 * items_host [max_items][4] receives (b, split, page_begin, page_end) for items
 * 0 .. *num_items-1, grouped by sequence in order; split_offsets_host [batch + 1]
 * receives the CSR offsets.  Both are plain host memory owned by the caller.
 * Errors: MLA_ERR_INVALID_ARG for null pointers, batch < 1, num_slots < 1 or a
 * seq_lens_host entry < 1; MLA_ERR_WORKSPACE when max_items is too small, in
 * which case *num_items is set to the capacity needed and nothing else is written. */
mla_status mla_plan_splits(const mla_dims* dims, int32_t batch, const int32_t* seq_lens_host,
                           int32_t num_slots, int32_t max_items, int32_t* items_host,
                           int32_t* split_offsets_host, int32_t* num_items);

/* mla_plan_splits for longest-first dispatch (host only, no HIP call,
 * deterministic).  Items and split offsets as mla_plan_splits writes them (the
 * same cover of every sequence, grouped by sequence in token order), but the
 * item size is chosen for dispatching the items longest first, and
 * order_host [max_items] receives that dispatch order: order_host[s] is the
 * item the s-th workgroup slot takes (a permutation of 0 .. *num_items-1,
 * items sorted by decreasing page count, equal sizes in item order).  The
 * simulation behind the size places dispatch slot s on XCD s % 8, as the
 * hardware places workgroups, and starts each XCD's items in order on its
 * num_slots / 8 slots.  With mixed lengths the longest items then start
 * first and the short ones fill the gaps at the end, which takes fewer,
 * larger items than in-order dispatch (fewer partials to merge).  Pass the
 * order to mla_decode_splitkv_ordered.
 * Errors: as for mla_plan_splits, plus MLA_ERR_INVALID_ARG for a null order_host. */
mla_status mla_plan_splits_ordered(const mla_dims* dims, int32_t batch, const int32_t* seq_lens_host,
                                   int32_t num_slots, int32_t max_items, int32_t* items_host,
                                   int32_t* split_offsets_host, int32_t* order_host,
                                   int32_t* num_items);

/* Upper bound on the number of items mla_plan_splits can produce for this batch:
 * sum over b of ceil(L_b / page_size).  Host only.  Returns -1 on bad arguments. */
int64_t mla_plan_max_items(const mla_dims* dims, int32_t batch, const int32_t* seq_lens_host);

/* Split-KV decode over the paged latent cache.
 * Page "DeepSeek-V2/V3：大模型的两张账" section "第一张账" (scores from the
 * transformed query and the cached latent; weighted sum in latent space) and RoPE
 * section (score = inner product of [content ; position] concatenations);
 * page "DeepSeek V2 技术解析" 2.1.1 (paged KV memory).
 * For work item w = (b, s, p0, p1), over tokens j in [p0*page_size, min(p1*page_size, L_b)):
 *   s_ij = softmax_scale * (q_abs[b][i] . kv_row_j)              (all d_latent + d_rope values)
 *   lse_part[w][i] = log sum_j exp(s_ij)
 *   o_part[w][i]   = sum_j exp(s_ij - lse_part[w][i]) * kv_row_j[0:d_latent]
 * Rows of unused cache slots are never read.
 * Errors: MLA_ERR_INVALID_ARG for null pointers, batch/num_items/num_pages/
 * max_pages_per_seq < 1 or misalignment; MLA_ERR_UNSUPPORTED for shapes out of range. */
mla_status mla_decode_splitkv(const mla_dims* dims, int32_t batch, const void* q_abs,
                              const void* kv_cache, int32_t num_pages, const int32_t* block_table,
                              int32_t max_pages_per_seq, const int32_t* seq_lens,
                              const int32_t* items, int32_t num_items, float* o_part,
                              float* lse_part, void* stream);

/* mla_decode_splitkv with a dispatch order: workgroup slot s decodes item
 * order[s] (device int32 [num_items], a permutation of 0 .. num_items-1, e.g.
 * from mla_plan_splits_ordered).  Partials are written at their item's index,
 * so o_part and lse_part are bit-identical to mla_decode_splitkv's on the same
 * items; only the time at which each item runs changes.  The order is taken on
 * trust (a value outside [0, num_items) is undefined behaviour); on shapes off
 * the gfx950 fast path it is ignored.
 * Errors: as for mla_decode_splitkv, plus MLA_ERR_INVALID_ARG for a null or
 * misaligned order. */
mla_status mla_decode_splitkv_ordered(const mla_dims* dims, int32_t batch, const void* q_abs,
                                      const void* kv_cache, int32_t num_pages,
                                      const int32_t* block_table, int32_t max_pages_per_seq,
                                      const int32_t* seq_lens, const int32_t* items,
                                      int32_t num_items, const int32_t* order, float* o_part,
                                      float* lse_part, void* stream);

/* Split-KV decode with q_len query tokens per sequence (speculative or chunked
 * decode: the newest q_len tokens of each sequence, already in the cache, are
 * decoded at once).  Page "DeepSeek V2 技术解析" 2.2.1.2 (the query of a step
 * sees only the tokens up to the one being predicted); the rest as for
 * mla_decode_splitkv.  Query token t of sequence b sits at position
 * L_b - q_len + t and sees cache rows j <= L_b - q_len + t.  For item w and token t:
 *   s_ij = softmax_scale * (q_abs[b][t][i] . kv_row_j),  j in [p0*page_size,
 *          min(p1*page_size, L_b - q_len + t + 1))
 *   lse_part[w][t][i], o_part[w][t][i] as for mla_decode_splitkv over those j;
 *   an item none of whose rows the token sees gives lse_part = -inf and o_part = 0
 *   (weight 0 in the merge).
 * Layouts: q_abs [batch][q_len][n_heads][d_latent + d_rope] (the rows of
 * mla_absorb_q called on batch * q_len rows); o_part [num_items][q_len][n_heads]
 * [d_latent] float32; lse_part [num_items][q_len][n_heads] float32.  Items and
 * the cache as for mla_decode_splitkv; q_len = 1 is mla_decode_splitkv.
 * Device data is not checked: every L_b must be >= q_len (a token that sees no
 * row has no defined output).
 * Errors: as for mla_decode_splitkv, plus MLA_ERR_INVALID_ARG for q_len < 1. */
mla_status mla_decode_splitkv_multi(const mla_dims* dims, int32_t batch, int32_t q_len,
                                    const void* q_abs, const void* kv_cache, int32_t num_pages,
                                    const int32_t* block_table, int32_t max_pages_per_seq,
                                    const int32_t* seq_lens, const int32_t* items,
                                    int32_t num_items, float* o_part, float* lse_part,
                                    void* stream);

/* Merge the work items of every sequence (exact softmax algebra over disjoint
 * token sets): M = max_s lse_s, w_s = exp(lse_s - M),
 * o_latent = sum_s w_s o_s / sum_s w_s, lse = M + log sum_s w_s.
 * `lse` may be NULL.  split_offsets is a device copy of the planner's array.
 * Errors: MLA_ERR_INVALID_ARG for null pointers, batch < 1 or misalignment. */
mla_status mla_combine(const mla_dims* dims, int32_t batch, const int32_t* split_offsets,
                       const float* o_part, const float* lse_part, float* o_latent, float* lse,
                       void* stream);

/* mla_combine for the partials of mla_decode_splitkv_multi: row (b, t) merges
 * o_part[w][t] over the items w of sequence b.  o_latent [batch][q_len][n_heads]
 * [d_latent] float32, lse [batch][q_len][n_heads] float32 or NULL.
 * Errors: as for mla_combine, plus MLA_ERR_INVALID_ARG for q_len < 1. */
mla_status mla_combine_multi(const mla_dims* dims, int32_t batch, int32_t q_len,
                             const int32_t* split_offsets, const float* o_part,
                             const float* lse_part, float* o_latent, float* lse, void* stream);

/* Prefill through the naive path: per-head keys and values are materialised
 * from the latent, then the q_len newest tokens of each sequence (already in
 * the cache) attend causally to it.  Page "DeepSeek V2 技术解析" 2.2.1.1
 * (k^C = W^UK c^KV and v^C = W^UV c^KV recover per-head keys and values),
 * 2.2.1.2 (a query sees only the tokens up to its own) and 2.2.2 (key
 * [k^C ; RoPE(k^R)], query [q^C ; RoPE(q^R)]).  For sequence b of length L, head
 * i and token t at position p = L - q_len + t:
 *   K_j = [W^UK_i c_j ; kr_j]  (kr_j as cached, already rotated),  V_j = W^UV_i c_j
 *   q   = [q^C ; RoPE_p(q^R)]   (q^R not yet rotated: the call rotates it)
 *   out[b][t][i] = sum_{j <= p} softmax_j(softmax_scale * q . K_j) V_j   (float32)
 *   lse[b][t][i] = log sum_{j <= p} exp(softmax_scale * q . K_j)          (or NULL)
 * Layouts: q_nope [batch][q_len][n_heads][d_head] bf16; q_pe [batch][q_len]
 * [n_heads][d_rope] bf16; w_uk, w_uv [n_heads * d_head][d_latent] bf16; cache
 * and block table as for mla_decode_splitkv; out [batch][q_len][n_heads][d_head]
 * float32.  K^C and V^C are rounded to bf16 in `workspace` (device memory of at
 * least mla_prefill_workspace_bytes() bytes, 16-byte aligned, owned by the
 * caller; contents afterwards unspecified).  Supported shapes: bf16, d_latent
 * 512, d_rope 64, d_head 128, page 64, any head count.
 * Device data is not checked: every L_b must be >= q_len.
 * Errors: MLA_ERR_INVALID_ARG for null pointers, sizes < 1 or misalignment;
 * MLA_ERR_UNSUPPORTED for other shapes or sizes out of range; MLA_ERR_WORKSPACE
 * for a short workspace. */
mla_status mla_prefill_naive(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_nope,
                             const void* q_pe, const void* w_uk, const void* w_uv,
                             const void* kv_cache, int32_t num_pages, const int32_t* block_table,
                             int32_t max_pages_per_seq, const int32_t* seq_lens, void* workspace,
                             int64_t workspace_bytes, float* out, float* lse, void* stream);

/* Bytes of workspace mla_prefill_naive needs for this batch and block-table
 * width (K^C and V^C of every row the table can address, bf16); -1 on bad
 * arguments or an unsupported shape.  Host only. */
int64_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t max_pages_per_seq);

/* Split-KV decode with the log-sum-exp merge fused in: the o_latent and lse of
 * mla_combine from one launch (same items and split_offsets as the two calls).
 * Pages as for mla_decode_splitkv; the merge is the combine's exact algebra.
 * On the gfx950 fast path with 16 or 128 heads every workgroup writes its
 * partial to o_part / lse_part, releases it, and takes a ticket; the last
 * workgroup of a sequence (of a half of its heads, at 128 heads) merges the
 * partials in item order and resets the ticket.  A sequence with a single
 * item writes o_latent and lse directly.  With other head counts, and on
 * other shapes, this is mla_decode_splitkv followed by mla_combine on the
 * same stream (`tickets` is not touched).
 *   tickets   int32 [2 * batch] device memory, all zero on entry; every call
 *             leaves it zero (a call that fails before launching writes nothing)
 *   o_part, lse_part  scratch of the sizes mla_decode_splitkv needs; their
 *             contents afterwards are unspecified
 *   o_latent, lse     as for mla_combine (`lse` may be NULL)
 * Concurrent calls must not share `tickets`.
 * Errors: MLA_ERR_INVALID_ARG for null pointers, sizes < 1 or misalignment. */
mla_status mla_decode_merged(const mla_dims* dims, int32_t batch, const void* q_abs,
                             const void* kv_cache, int32_t num_pages, const int32_t* block_table,
                             int32_t max_pages_per_seq, const int32_t* seq_lens,
                             const int32_t* items, int32_t num_items,
                             const int32_t* split_offsets, float* o_part, float* lse_part,
                             int32_t* tickets, float* o_latent, float* lse, void* stream);

/* Map the latent-space result out through W^UV: out[b][i] = W^UV_i o_latent[b][i].
 * Page "DeepSeek V2 技术解析" 2.2.1.1 (W^UV absorbed on the output side) and page
 * "DeepSeek-V2/V3：大模型的两张账" "第一张账" (latent-space result mapped out).
 * float32 o_latent is split into two bf16 terms (hi + lo) on the fast path, so
 * the product carries about 16 significant bits of o_latent.
 * Errors: MLA_ERR_INVALID_ARG for null pointers, batch < 1 or misalignment. */
mla_status mla_out_proj(const mla_dims* dims, int32_t batch, const float* o_latent,
                        const void* w_uv, float* out, void* stream);

/* mla_combine_multi followed by mla_out_proj on the batch * q_len rows, in one
 * launch on the gfx950 fast path: each workgroup merges the partials of its rows
 * (the combine's arithmetic and order, so o_latent is bit-identical to
 * mla_combine's) and feeds the merged rows to the W^UV product without writing
 * them out first.  Cites as mla_combine and mla_out_proj.  A workgroup takes
 * 32, 16, 8 or 4 query rows of one head (fewer when 32 would leave CUs idle); the
 * result does not depend on that choice.
 *   split_offsets, o_part, lse_part  as for mla_combine_multi (q_len = 1: as for
 *             mla_combine)
 *   out       float32 [batch][q_len][n_heads][d_head]
 *   o_latent  float32 [batch][q_len][n_heads][d_latent] or NULL on the fast path;
 *             on other shapes it is required (the two kernels run with it between them)
 *   lse       float32 [batch][q_len][n_heads] or NULL
 * Errors: MLA_ERR_INVALID_ARG for null required pointers, batch or q_len < 1 or
 * misalignment; MLA_ERR_UNSUPPORTED for sizes out of range or a NULL o_latent
 * on a shape off the fast path. */
mla_status mla_combine_out_proj(const mla_dims* dims, int32_t batch, int32_t q_len,
                                const int32_t* split_offsets, const float* o_part,
                                const float* lse_part, const void* w_uv, float* out,
                                float* o_latent, float* lse, void* stream);

/* Write the token being decoded into the paged latent cache, one per sequence.
 * Page "DeepSeek V2 技术解析" 2.2.1.1 (only c^KV = W^DKV h_t is kept for the keys
 * and values) and 2.2.2 (k^R_t = W^KR h_t, shared by the heads, cached after the
 * rotation R_t); page "DeepSeek-V2/V3：大模型的两张账" "第一张账" (normalised latent).
 * For every b, with p = positions[b]:
 *   c  = W^DKV h[b]; if rms_norm: c = c / sqrt(mean(c^2) + eps)   (no gain)
 *   kr = RoPE_p(W^KR h[b])  (pairs (2k, 2k+1), angle p * rope_base^(-2k/d_rope) in float64)
 *   kv_cache row (page block_table[b][p / page_size], slot p % page_size) = [c | kr],
 *   rounded to dtype (nearest, ties to even).  No other byte of the cache changes.
 * Layouts: h [batch][d_model] dtype; w_dkv [d_latent][d_model] dtype; w_kr
 * [d_rope][d_model] dtype (both map column vectors); positions [batch] int32;
 * kv_cache, block_table as for mla_decode_splitkv.  Products accumulate in float32.
 * workspace: device memory of at least mla_append_kv_workspace_bytes() bytes,
 * 16-byte aligned, owned by the caller; its contents afterwards are unspecified.
 * Device data is not checked: p must lie in [0, max_pages_per_seq * page_size)
 * and the block-table entry in [0, num_pages); two sequences must not write the
 * same slot.
 * Errors: MLA_ERR_INVALID_ARG for null pointers, sizes < 1, misalignment or a
 * non-positive eps with rms_norm set; MLA_ERR_WORKSPACE for a short workspace. */
mla_status mla_append_kv(const mla_dims* dims, int32_t d_model, int32_t batch, const void* h,
                         const void* w_dkv, const void* w_kr, const int32_t* positions,
                         int32_t rms_norm, float eps, void* kv_cache, int32_t num_pages,
                         const int32_t* block_table, int32_t max_pages_per_seq, void* workspace,
                         int64_t workspace_bytes, void* stream);

/* Bytes of workspace mla_append_kv needs; -1 on bad arguments.  Host only. */
int64_t mla_append_kv_workspace_bytes(const mla_dims* dims, int32_t d_model, int32_t batch);

/* mla_append_kv without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (minus the workspace), same
 * kernels and the same result bits as mla_append_kv.  The K-slice partial sums
 * go to a static device buffer of the library (mla_append_kv_noalloc_max_bytes()
 * = 8 MiB per device, held until the process ends); the call allocates
 * nothing.  Its device address is looked up once per device, on the first call
 * made with that device current.  Every element of the buffer that a call
 * reads is written earlier in the same call, so nothing needs clearing between
 * calls.  All calls on one device share the buffer: calls that can overlap in
 * time on one device (different streams, or different host threads without
 * ordering) race and must not be made.
 * Errors: as for mla_append_kv; MLA_ERR_WORKSPACE when
 * mla_append_kv_workspace_bytes(dims, d_model, batch) exceeds the buffer
 * (e.g. more than 455 tokens at d_model 5120 with d_c + d_h^R = 576);
 * MLA_ERR_HIP if the buffer's address cannot be found on the current device. */
mla_status mla_append_kv_noalloc(const mla_dims* dims, int32_t d_model, int32_t batch, const void* h,
                                 const void* w_dkv, const void* w_kr, const int32_t* positions,
                                 int32_t rms_norm, float eps, void* kv_cache, int32_t num_pages,
                                 const int32_t* block_table, int32_t max_pages_per_seq,
                                 void* stream);

/* Size in bytes of mla_append_kv_noalloc's static buffer (per device). */
int64_t mla_append_kv_noalloc_max_bytes(void);

/* Debug check of the device data the decode and prefill entry points take on
 * trust.  Page "DeepSeek V2 技术解析" 2.1.1 (paged KV memory): sequence b reads
 * pages block_table[b][0 .. ceil(L_b / page_size) - 1], which must lie in
 * [0, num_pages), with L_b = seq_lens[b] in [min_len, max_pages_per_seq * page_size]
 * (min_len = 1 for mla_decode_splitkv and mla_decode_merged, q_len for
 * mla_decode_splitkv_multi and mla_prefill_naive).
 * Writes result[0] = the number of bad values (one per length out of range,
 * whose entries are then not looked at, plus one per entry out of range among
 * the pages a good length uses) and result[1] = the smallest b with a bad value,
 * or -1.  result: device int32[2], owned by the caller, need not be cleared.
 * One workgroup: cheap next to a decode step, but not free; meant for debugging.
 * Entries past a sequence's pages are not looked at.
 * Errors: MLA_ERR_INVALID_ARG for null pointers, batch/min_len/num_pages/
 * max_pages_per_seq < 1 or misalignment. */
mla_status mla_check_paging(const mla_dims* dims, int32_t batch, int32_t min_len,
                            const int32_t* seq_lens, int32_t num_pages, const int32_t* block_table,
                            int32_t max_pages_per_seq, int32_t* result, void* stream);

/* Number of workgroups of the 128-head fast decode (each takes one half of a
 * work item's heads for one query token) that recomputed their item against
 * exact score maxima (the scores rose past the reference by more than 64
 * log2 units within one window of 8 slices) on the current device since the
 * count was last reset; with reset != 0 the count goes back to zero after it
 * is read.  For monitoring and tests: the
 * call copies a device counter synchronously.  Pages as for mla_decode_splitkv
 * (the softmax of one head over the item's tokens).
 * Errors: MLA_ERR_INVALID_ARG for a null count_host; MLA_ERR_HIP if the copy fails. */
mla_status mla_decode_exact_pass_count(int32_t reset, uint64_t* count_host);

/* Text of the last HIP error that made a libmla call on this thread return
 * MLA_ERR_HIP ("" if none).  Valid until the next libmla call on the thread. */
const char* mla_last_hip_error(void);

/* Static description of a status code (never NULL). */
const char* mla_status_string(mla_status status);

/* MLA_VERSION of the built library. */
int32_t mla_version(void);

/* 1 when the shape takes the gfx950 fast path, 0 when it takes the
 * straightforward kernels, negative status when it is rejected. */
int32_t mla_fast_path(const mla_dims* dims);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
