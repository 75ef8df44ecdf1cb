// Internal declarations shared by the libmla translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// Fast-path shape: bf16, d_c 512, d_h^R 64, d_h 128, 64-token pages.
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kDq = kDc + kDr;  // 576 values per cached row / absorbed query
constexpr int kDh = 128;
constexpr int kPage = 64;

bool is_fast_shape(const mla_dims& d);

// Launchers: enqueue on `stream`, return the launch status.
hipError_t absorb_generic(const mla_dims& d, int batch, const void* q_nope, const void* q_pe,
                          const int32_t* positions, const void* w_uk, void* q_abs,
                          hipStream_t stream);
hipError_t decode_generic(const mla_dims& d, int q_len, const void* q_abs, const void* kv_cache,
                          const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                          const int32_t* items, int num_items, float* o_part, float* lse_part,
                          hipStream_t stream);
hipError_t combine_generic(const mla_dims& d, int batch, int q_len, const int32_t* split_offsets,
                           const float* o_part, const float* lse_part, float* o_latent, float* lse,
                           hipStream_t stream);
hipError_t out_proj_generic(const mla_dims& d, int batch, const float* o_latent, const void* w_uv,
                            float* out, hipStream_t stream);

// Grid sizes of the fast dense kernels (grid y is at most 65535): workgroups
// along the rows for absorb and out_proj, and the rows per workgroup the fused
// merge + out_proj picks.
int64_t absorb_fast_groups(int64_t batch);
int64_t out_proj_fast_groups(int64_t rows);
int combine_out_proj_rows_per_group(int n_heads, int64_t rows);
hipError_t absorb_fast(const mla_dims& d, int batch, const void* q_nope, const void* q_pe,
                       const int32_t* positions, const void* w_uk, void* q_abs,
                       hipStream_t stream);
// With tickets == nullptr: partials only.  Otherwise also the merge of every
// sequence's partials into o_latent / lse_out (split_offsets as for combine;
// q_len 1 only).  q_len query tokens per sequence: q_abs rows b * q_len + t,
// partial rows item * q_len + t.
// Items the 128-head fast decode redid against exact maxima on the current
// device since the last reset (synchronous copies of a device counter).
hipError_t exact_pass_count(uint64_t* count, bool reset);
// order: null, or the item each dispatch slot takes (a permutation of the items).
hipError_t decode_fast(const mla_dims& d, int q_len, const void* q_abs, const void* kv_cache,
                       const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                       const int32_t* items, int num_items, const int32_t* order, float* o_part,
                       float* lse_part,
                       const int32_t* split_offsets, int32_t* tickets, float* o_latent,
                       float* lse_out, hipStream_t stream);
hipError_t combine_fast(const mla_dims& d, int batch, int q_len, const int32_t* split_offsets,
                        const float* o_part, const float* lse_part, float* o_latent, float* lse,
                        hipStream_t stream);
hipError_t out_proj_fast(const mla_dims& d, int batch, const float* o_latent, const void* w_uv,
                         float* out, hipStream_t stream);
// combine + out_proj in one launch (the merged o~ staged in LDS, never read
// back); o_latent and lse are written when not null.
hipError_t combine_out_proj_fast(const mla_dims& d, int batch, int q_len, const int32_t* split_offsets,
                                 const float* o_part, const float* lse_part, const void* w_uv,
                                 float* out, float* o_latent, float* lse, hipStream_t stream);

// Prefill through the materialised-K/V path (bf16, d_c 512, d_h^R 64, d_h 128,
// 64-token pages, any head count).
bool is_prefill_shape(const mla_dims& d);
int64_t prefill_workspace_bytes(const mla_dims& d, int batch, int max_pages);
hipError_t prefill_naive(const mla_dims& d, int batch, int q_len, const void* q_nope, const void* q_pe,
                         const void* w_uk, const void* w_uv, const void* kv_cache,
                         const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                         void* workspace, float* out, float* lse, hipStream_t stream);

// Cache write of one token per sequence (append.hip); `ws` holds
// append_slices(d_model) x batch x (d_latent + d_rope) floats.
int append_slices(int d_model);
// The static scratch of mla_append_kv_noalloc: its size, and its device
// address on the current device (looked up once per device).
constexpr int64_t kAppendScratchBytes = int64_t{8} << 20;
hipError_t scratch_on_current_device(float** out);
hipError_t append_kv(const mla_dims& d, int d_model, int batch, const void* h, const void* w_dkv,
                     const void* w_kr, const int32_t* positions, bool rms_norm, float eps,
                     void* kv_cache, const int32_t* block_table, int max_pages, float* ws,
                     hipStream_t stream);

// Debug check of seq_lens and the block-table entries they address (check.hip):
// result[0] = bad values, result[1] = first bad sequence or -1.
hipError_t check_paging(const mla_dims& d, int batch, int min_len, const int32_t* seq_lens,
                        const int32_t* block_table, int max_pages, int num_pages,
                        int32_t* result, hipStream_t stream);

// Host planner (plan.cpp).
// order: null, or [max_items] to receive the longest-first dispatch order (the
// item size is then chosen for that order).
mla_status plan_splits(int page_size, int batch, const int32_t* seq_lens, int num_slots,
                       int max_items, int32_t* items, int32_t* split_offsets, int32_t* num_items,
                       int n_heads, int32_t* order = nullptr);
int64_t plan_max_items(int page_size, int batch, const int32_t* seq_lens);

}  // namespace mla
