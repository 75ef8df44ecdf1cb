// C-ABI entry points of libmla: argument checks (host, before any HIP call)
// and dispatch to the gfx950 fast path or the straightforward kernels.
#include <math.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {

bool is_fast_shape(const mla_dims& d) {
  return d.dtype == MLA_BF16 && d.d_latent == kDc && d.d_rope == kDr && d.d_head == kDh &&
         d.page_size == kPage && d.n_heads % 16 == 0;
}

namespace {

// Workgroups the decode gives one work item and query token: the fast path
// takes 16 heads in one workgroup and otherwise up to 64 heads per workgroup
// (ceil(H / 64)); the straightforward kernels take a whole item.
int decode_groups(const mla_dims& d) {
  if (!is_fast_shape(d) || d.n_heads == 16) return 1;
  return (d.n_heads + 63) / 64;
}

mla_status check_dims(const mla_dims* d) {
  if (!d) return MLA_ERR_INVALID_ARG;
  if (d->dtype != MLA_BF16 && d->dtype != MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (d->n_heads < 1 || d->d_head < 1 || d->d_latent < 1 || d->d_rope < 0 ||
      (d->d_rope & 1) != 0 || d->page_size < 1)
    return MLA_ERR_INVALID_ARG;
  if (!isfinite(d->softmax_scale) || !isfinite(d->rope_base) || !(d->rope_base > 0.0))
    return MLA_ERR_INVALID_ARG;
  if (d->n_heads > 1024 || d->d_head > 256 || d->d_latent > 1024 || d->d_rope > 128 ||
      d->page_size > 1024)
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

thread_local const char* t_last_hip_error = "";

inline mla_status launched(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  t_last_hip_error = hipGetErrorString(e);
  return MLA_ERR_HIP;
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MLA_ERR_WORKSPACE: return "capacity too small";
    case MLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t mla_version(void) { return MLA_VERSION; }

const char* mla_last_hip_error(void) { return t_last_hip_error; }

int32_t mla_fast_path(const mla_dims* d) {
  const mla_status s = check_dims(d);
  if (s != MLA_OK) return s;
  return is_fast_shape(*d) ? 1 : 0;
}

mla_status mla_absorb_q(const mla_dims* dims, int32_t batch, const void* q_nope, const void* q_pe,
                        const int32_t* positions, const void* w_uk, void* q_abs, void* stream) {
  mla_status s = check_dims(dims);
  if (s != MLA_OK) return s;
  if (batch < 1 || !q_nope || !q_pe || !positions || !w_uk || !q_abs) return MLA_ERR_INVALID_ARG;
  if (!al16(q_nope) || !al16(q_pe) || !al16(w_uk) || !al16(q_abs) || !al4(positions))
    return MLA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(batch) * dims->n_heads > (int64_t{1} << 31)) return MLA_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // drop an error left on this thread by an earlier, unrelated call
  if (is_fast_shape(*dims)) {
    if (absorb_fast_groups(batch) > 65535) return MLA_ERR_UNSUPPORTED;
    return launched(absorb_fast(*dims, batch, q_nope, q_pe, positions, w_uk, q_abs, st));
  }
  if (batch > 65535) return MLA_ERR_UNSUPPORTED;
  return launched(absorb_generic(*dims, batch, q_nope, q_pe, positions, w_uk, q_abs, st));
}

int64_t mla_plan_max_items(const mla_dims* dims, int32_t batch, const int32_t* seq_lens_host) {
  if (check_dims(dims) != MLA_OK) return -1;
  return plan_max_items(dims->page_size, batch, seq_lens_host);
}

mla_status mla_plan_splits(const mla_dims* dims, int32_t batch, const int32_t* seq_lens_host,
                           int32_t num_slots, int32_t max_items, int32_t* items_host,
                           int32_t* split_offsets_host, int32_t* num_items) {
  mla_status s = check_dims(dims);
  if (s != MLA_OK) return s;
  // The fast decode gives every item decode_groups() workgroups (two at 128
  // heads, one per half of the heads), so about num_slots / that many items
  // fill the machine.
  const int per_item = decode_groups(*dims);
  const int slots = num_slots >= per_item ? num_slots / per_item : num_slots;
  return plan_splits(dims->page_size, batch, seq_lens_host, slots, max_items, items_host,
                     split_offsets_host, num_items, dims->n_heads);
}

mla_status mla_plan_splits_ordered(const mla_dims* dims, int32_t batch, const int32_t* seq_lens_host,
                                   int32_t num_slots, int32_t max_items, int32_t* items_host,
                                   int32_t* split_offsets_host, int32_t* order_host,
                                   int32_t* num_items) {
  mla_status s = check_dims(dims);
  if (s != MLA_OK) return s;
  if (!order_host) return MLA_ERR_INVALID_ARG;
  const int per_item = decode_groups(*dims);
  const int slots = num_slots >= per_item ? num_slots / per_item : num_slots;
  return plan_splits(dims->page_size, batch, seq_lens_host, slots, max_items, items_host,
                     split_offsets_host, num_items, dims->n_heads, order_host);
}

namespace {

mla_status decode_splitkv_impl(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_abs,
                               const void* kv_cache, int32_t num_pages, const int32_t* block_table,
                               int32_t max_pages_per_seq, const int32_t* seq_lens,
                               const int32_t* items, int32_t num_items, const int32_t* order,
                               float* o_part, float* lse_part, void* stream) {
  mla_status s = check_dims(dims);
  if (s != MLA_OK) return s;
  if (batch < 1 || q_len < 1 || num_pages < 1 || max_pages_per_seq < 1 || num_items < 1)
    return MLA_ERR_INVALID_ARG;
  if (!q_abs || !kv_cache || !block_table || !seq_lens || !items || !o_part || !lse_part)
    return MLA_ERR_INVALID_ARG;
  if (!al16(q_abs) || !al16(kv_cache) || !al16(o_part) || !al4(lse_part) || !al4(block_table) ||
      !al4(seq_lens) || !al4(items) || (order && !al4(order)))
    return MLA_ERR_INVALID_ARG;
  // partial rows and workgroup counts stay within 32-bit grid limits
  if (static_cast<int64_t>(num_items) * q_len * decode_groups(*dims) > INT32_MAX ||
      static_cast<int64_t>(batch) * q_len * dims->n_heads > (int64_t{1} << 31))
    return MLA_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // drop an error left on this thread by an earlier, unrelated call
  if (is_fast_shape(*dims))
    return launched(decode_fast(*dims, q_len, q_abs, kv_cache, block_table, max_pages_per_seq,
                                seq_lens, items, num_items, order, o_part, lse_part, nullptr,
                                nullptr, nullptr, nullptr, st));
  return launched(decode_generic(*dims, q_len, q_abs, kv_cache, block_table, max_pages_per_seq,
                                 seq_lens, items, num_items, o_part, lse_part, st));
}

mla_status combine_impl(const mla_dims* dims, int32_t batch, int32_t q_len,
                        const int32_t* split_offsets, const float* o_part, const float* lse_part,
                        float* o_latent, float* lse, void* stream) {
  mla_status s = check_dims(dims);
  if (s != MLA_OK) return s;
  if (batch < 1 || q_len < 1 || !split_offsets || !o_part || !lse_part || !o_latent)
    return MLA_ERR_INVALID_ARG;
  if (!al16(o_part) || !al16(o_latent) || !al4(lse_part) || !al4(split_offsets) ||
      (lse && !al4(lse)))
    return MLA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(batch) * q_len * dims->n_heads > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // drop an error left on this thread by an earlier, unrelated call
  if (is_fast_shape(*dims))
    return launched(combine_fast(*dims, batch, q_len, split_offsets, o_part, lse_part, o_latent, lse,
                                 st));
  if (static_cast<int64_t>(batch) * q_len > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  return launched(combine_generic(*dims, batch, q_len, split_offsets, o_part, lse_part, o_latent,
                                  lse, st));
}

}  // namespace

mla_status mla_decode_splitkv(const mla_dims* dims, int32_t batch, const void* q_abs,
                              const void* kv_cache, int32_t num_pages, const int32_t* block_table,
                              int32_t max_pages_per_seq, const int32_t* seq_lens,
                              const int32_t* items, int32_t num_items, float* o_part,
                              float* lse_part, void* stream) {
  return decode_splitkv_impl(dims, batch, 1, q_abs, kv_cache, num_pages, block_table,
                             max_pages_per_seq, seq_lens, items, num_items, nullptr, o_part, lse_part,
                             stream);
}

mla_status mla_decode_splitkv_ordered(const mla_dims* dims, int32_t batch, const void* q_abs,
                                      const void* kv_cache, int32_t num_pages,
                                      const int32_t* block_table, int32_t max_pages_per_seq,
                                      const int32_t* seq_lens, const int32_t* items,
                                      int32_t num_items, const int32_t* order, float* o_part,
                                      float* lse_part, void* stream) {
  if (!order) return MLA_ERR_INVALID_ARG;
  return decode_splitkv_impl(dims, batch, 1, q_abs, kv_cache, num_pages, block_table,
                             max_pages_per_seq, seq_lens, items, num_items, order, o_part, lse_part,
                             stream);
}

mla_status mla_decode_splitkv_multi(const mla_dims* dims, int32_t batch, int32_t q_len,
                                    const void* q_abs, const void* kv_cache, int32_t num_pages,
                                    const int32_t* block_table, int32_t max_pages_per_seq,
                                    const int32_t* seq_lens, const int32_t* items,
                                    int32_t num_items, float* o_part, float* lse_part,
                                    void* stream) {
  return decode_splitkv_impl(dims, batch, q_len, q_abs, kv_cache, num_pages, block_table,
                             max_pages_per_seq, seq_lens, items, num_items, nullptr, o_part, lse_part,
                             stream);
}

mla_status mla_decode_merged(const mla_dims* dims, int32_t batch, const void* q_abs,
                             const void* kv_cache, int32_t num_pages, const int32_t* block_table,
                             int32_t max_pages_per_seq, const int32_t* seq_lens,
                             const int32_t* items, int32_t num_items,
                             const int32_t* split_offsets, float* o_part, float* lse_part,
                             int32_t* tickets, float* o_latent, float* lse, void* stream) {
  mla_status s = check_dims(dims);
  if (s != MLA_OK) return s;
  if (batch < 1 || num_pages < 1 || max_pages_per_seq < 1 || num_items < 1) return MLA_ERR_INVALID_ARG;
  if (!q_abs || !kv_cache || !block_table || !seq_lens || !items || !split_offsets || !o_part ||
      !lse_part || !tickets || !o_latent)
    return MLA_ERR_INVALID_ARG;
  if (!al16(q_abs) || !al16(kv_cache) || !al16(o_part) || !al16(o_latent) || !al4(lse_part) ||
      !al4(block_table) || !al4(seq_lens) || !al4(items) || !al4(split_offsets) || !al4(tickets) ||
      (lse && !al4(lse)))
    return MLA_ERR_INVALID_ARG;
  // partial rows and workgroup counts stay within 32-bit grid limits
  if (static_cast<int64_t>(num_items) * decode_groups(*dims) > INT32_MAX ||
      static_cast<int64_t>(batch) * dims->n_heads > (int64_t{1} << 31))
    return MLA_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // drop an error left on this thread by an earlier, unrelated call
  if (is_fast_shape(*dims) && (dims->n_heads == 16 || dims->n_heads == 128))
    return launched(decode_fast(*dims, 1, q_abs, kv_cache, block_table, max_pages_per_seq,
                                seq_lens, items, num_items, nullptr, o_part, lse_part, split_offsets,
                                tickets, o_latent, lse, st));
  if (is_fast_shape(*dims)) {
    // other head counts: the fast decode and the fast merge as two launches
    // (the ticket array holds two counters per sequence, as many as 128
    // heads use); `tickets` is left untouched
    mla_status r = launched(decode_fast(*dims, 1, q_abs, kv_cache, block_table, max_pages_per_seq,
                                        seq_lens, items, num_items, nullptr, o_part, lse_part,
                                        nullptr, nullptr, nullptr, nullptr, st));
    if (r != MLA_OK) return r;
    return launched(combine_fast(*dims, batch, 1, split_offsets, o_part, lse_part, o_latent, lse, st));
  }
  mla_status r = launched(decode_generic(*dims, 1, q_abs, kv_cache, block_table, max_pages_per_seq,
                                         seq_lens, items, num_items, o_part, lse_part, st));
  if (r != MLA_OK) return r;
  return launched(combine_generic(*dims, batch, 1, split_offsets, o_part, lse_part, o_latent, lse,
                                  st));
}

mla_status mla_combine(const mla_dims* dims, int32_t batch, const int32_t* split_offsets,
                       const float* o_part, const float* lse_part, float* o_latent, float* lse,
                       void* stream) {
  return combine_impl(dims, batch, 1, split_offsets, o_part, lse_part, o_latent, lse, stream);
}

mla_status mla_combine_multi(const mla_dims* dims, int32_t batch, int32_t q_len,
                             const int32_t* split_offsets, const float* o_part,
                             const float* lse_part, float* o_latent, float* lse, void* stream) {
  return combine_impl(dims, batch, q_len, split_offsets, o_part, lse_part, o_latent, lse, stream);
}

mla_status mla_decode_exact_pass_count(int32_t reset, uint64_t* count_host) {
  if (!count_host) return MLA_ERR_INVALID_ARG;
  (void)hipGetLastError();  // drop an error left on this thread by an earlier, unrelated call
  return launched(exact_pass_count(count_host, reset != 0));
}

mla_status mla_check_paging(const mla_dims* dims, int32_t batch, int32_t min_len,
                            const int32_t* seq_lens, int32_t num_pages, const int32_t* block_table,
                            int32_t max_pages_per_seq, int32_t* result, void* stream) {
  mla_status s = check_dims(dims);
  if (s != MLA_OK) return s;
  if (batch < 1 || min_len < 1 || num_pages < 1 || max_pages_per_seq < 1) return MLA_ERR_INVALID_ARG;
  if (!seq_lens || !block_table || !result) return MLA_ERR_INVALID_ARG;
  if (!al4(seq_lens) || !al4(block_table) || !al4(result)) return MLA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // drop an error left on this thread by an earlier, unrelated call
  return launched(check_paging(*dims, batch, min_len, seq_lens, block_table, max_pages_per_seq,
                               num_pages, result, st));
}

int64_t mla_append_kv_workspace_bytes(const mla_dims* dims, int32_t d_model, int32_t batch) {
  if (check_dims(dims) != MLA_OK || d_model < 1 || batch < 1) return -1;
  return static_cast<int64_t>(append_slices(d_model)) * batch * (dims->d_latent + dims->d_rope) *
         static_cast<int64_t>(sizeof(float));
}

mla_status mla_append_kv(const mla_dims* dims, int32_t d_model, int32_t batch, const void* h,
                         const void* w_dkv, const void* w_kr, const int32_t* positions,
                         int32_t rms_norm, float eps, void* kv_cache, int32_t num_pages,
                         const int32_t* block_table, int32_t max_pages_per_seq, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  mla_status s = check_dims(dims);
  if (s != MLA_OK) return s;
  if (d_model < 1 || batch < 1 || num_pages < 1 || max_pages_per_seq < 1) return MLA_ERR_INVALID_ARG;
  if (!h || !w_dkv || !w_kr || !positions || !kv_cache || !block_table || !workspace)
    return MLA_ERR_INVALID_ARG;
  if (rms_norm && !(eps > 0.f && isfinite(eps))) return MLA_ERR_INVALID_ARG;
  if (!al16(h) || !al16(w_dkv) || !al16(w_kr) || !al16(kv_cache) || !al16(workspace) ||
      !al4(positions) || !al4(block_table))
    return MLA_ERR_INVALID_ARG;
  if (d_model > (1 << 20) || batch > 65535) return MLA_ERR_UNSUPPORTED;
  if (workspace_bytes < mla_append_kv_workspace_bytes(dims, d_model, batch)) return MLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // drop an error left on this thread by an earlier, unrelated call
  return launched(append_kv(*dims, d_model, batch, h, w_dkv, w_kr, positions, rms_norm != 0, eps,
                            kv_cache, block_table, max_pages_per_seq,
                            static_cast<float*>(workspace), st));
}

mla_status mla_append_kv_noalloc(const mla_dims* dims, int32_t d_model, int32_t batch, const void* h,
                                 const void* w_dkv, const void* w_kr, const int32_t* positions,
                                 int32_t rms_norm, float eps, void* kv_cache, int32_t num_pages,
                                 const int32_t* block_table, int32_t max_pages_per_seq,
                                 void* stream) {
  mla_status s = check_dims(dims);
  if (s != MLA_OK) return s;
  if (d_model < 1 || batch < 1 || num_pages < 1 || max_pages_per_seq < 1) return MLA_ERR_INVALID_ARG;
  if (!h || !w_dkv || !w_kr || !positions || !kv_cache || !block_table) return MLA_ERR_INVALID_ARG;
  if (rms_norm && !(eps > 0.f && isfinite(eps))) return MLA_ERR_INVALID_ARG;
  if (!al16(h) || !al16(w_dkv) || !al16(w_kr) || !al16(kv_cache) || !al4(positions) ||
      !al4(block_table))
    return MLA_ERR_INVALID_ARG;
  if (d_model > (1 << 20) || batch > 65535) return MLA_ERR_UNSUPPORTED;
  if (mla_append_kv_workspace_bytes(dims, d_model, batch) > kAppendScratchBytes) return MLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // drop an error left on this thread by an earlier, unrelated call
  float* ws = nullptr;
  mla_status r = launched(scratch_on_current_device(&ws));
  if (r != MLA_OK) return r;
  return launched(append_kv(*dims, d_model, batch, h, w_dkv, w_kr, positions, rms_norm != 0, eps,
                            kv_cache, block_table, max_pages_per_seq, ws, st));
}

int64_t mla_append_kv_noalloc_max_bytes(void) { return kAppendScratchBytes; }

mla_status mla_out_proj(const mla_dims* dims, int32_t batch, const float* o_latent,
                        const void* w_uv, float* out, void* stream) {
  mla_status s = check_dims(dims);
  if (s != MLA_OK) return s;
  if (batch < 1 || !o_latent || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  if (!al16(o_latent) || !al16(w_uv) || !al16(out)) return MLA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // drop an error left on this thread by an earlier, unrelated call
  if (is_fast_shape(*dims)) {
    if (out_proj_fast_groups(batch) > 65535) return MLA_ERR_UNSUPPORTED;
    return launched(out_proj_fast(*dims, batch, o_latent, w_uv, out, st));
  }
  if (batch > 65535) return MLA_ERR_UNSUPPORTED;
  return launched(out_proj_generic(*dims, batch, o_latent, w_uv, out, st));
}

int64_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t max_pages_per_seq) {
  if (check_dims(dims) != MLA_OK || batch < 1 || max_pages_per_seq < 1) return -1;
  if (!is_prefill_shape(*dims)) return -1;
  return prefill_workspace_bytes(*dims, batch, max_pages_per_seq);
}

mla_status mla_prefill_naive(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_nope,
                             const void* q_pe, const void* w_uk, const void* w_uv,
                             const void* kv_cache, int32_t num_pages, const int32_t* block_table,
                             int32_t max_pages_per_seq, const int32_t* seq_lens, void* workspace,
                             int64_t workspace_bytes, float* out, float* lse, void* stream) {
  mla_status s = check_dims(dims);
  if (s != MLA_OK) return s;
  if (batch < 1 || q_len < 1 || num_pages < 1 || max_pages_per_seq < 1) return MLA_ERR_INVALID_ARG;
  if (!q_nope || !q_pe || !w_uk || !w_uv || !kv_cache || !block_table || !seq_lens || !workspace ||
      !out)
    return MLA_ERR_INVALID_ARG;
  if (!al16(q_nope) || !al16(q_pe) || !al16(w_uk) || !al16(w_uv) || !al16(kv_cache) ||
      !al16(workspace) || !al16(out) || !al4(block_table) || !al4(seq_lens) || (lse && !al4(lse)))
    return MLA_ERR_INVALID_ARG;
  if (!is_prefill_shape(*dims)) return MLA_ERR_UNSUPPORTED;
  // the materialisation grid is (heads, batch); the attention's is 1-D
  if (batch > 65535 ||
      static_cast<int64_t>(batch) * q_len * dims->n_heads > (int64_t{1} << 31) ||
      static_cast<int64_t>(max_pages_per_seq) * 64 > (int64_t{1} << 24))
    return MLA_ERR_UNSUPPORTED;
  if (workspace_bytes < prefill_workspace_bytes(*dims, batch, max_pages_per_seq)) return MLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // drop an error left on this thread by an earlier, unrelated call
  return launched(prefill_naive(*dims, batch, q_len, q_nope, q_pe, w_uk, w_uv, kv_cache, block_table,
                                max_pages_per_seq, seq_lens, workspace, out, lse, st));
}

mla_status mla_combine_out_proj(const mla_dims* dims, int32_t batch, int32_t q_len,
                                const int32_t* split_offsets, const float* o_part,
                                const float* lse_part, const void* w_uv, float* out,
                                float* o_latent, float* lse, void* stream) {
  mla_status s = check_dims(dims);
  if (s != MLA_OK) return s;
  if (batch < 1 || q_len < 1 || !split_offsets || !o_part || !lse_part || !w_uv || !out)
    return MLA_ERR_INVALID_ARG;
  if (!al16(o_part) || !al4(lse_part) || !al4(split_offsets) || !al16(w_uv) || !al16(out) ||
      (o_latent && !al16(o_latent)) || (lse && !al4(lse)))
    return MLA_ERR_INVALID_ARG;
  const int64_t rows = static_cast<int64_t>(batch) * q_len;
  if (rows * dims->n_heads > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (is_fast_shape(*dims)) {
    const int R = combine_out_proj_rows_per_group(dims->n_heads, rows);
    if ((rows + R - 1) / R > 65535) return MLA_ERR_UNSUPPORTED;
    (void)hipGetLastError();  // drop an error left on this thread by an earlier, unrelated call
    return launched(combine_out_proj_fast(*dims, batch, q_len, split_offsets, o_part, lse_part, w_uv,
                                          out, o_latent, lse, st));
  }
  // other shapes: the two kernels, with o_latent as the buffer between them
  if (!o_latent) return MLA_ERR_UNSUPPORTED;
  if (rows > 65535) return MLA_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // drop an error left on this thread by an earlier, unrelated call
  mla_status r = launched(combine_generic(*dims, batch, q_len, split_offsets, o_part, lse_part,
                                          o_latent, lse, st));
  if (r != MLA_OK) return r;
  return launched(out_proj_generic(*dims, static_cast<int>(rows), o_latent, w_uv, out, st));
}

}  // extern "C"
