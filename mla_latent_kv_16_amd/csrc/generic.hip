// Straightforward kernels for any supported shape and for float32 storage.
//
// One workgroup per (row, head); float32 arithmetic throughout.  They serve
// shapes outside the gfx950 fast path (for example d_c 64, d_h^R 8, float32)
// and are not tuned.
#include <math.h>

#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;

__device__ float block_reduce_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ float block_reduce_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < kThreads / 64; ++i) r += red[i];
  return r;
}

// q_abs[b][h] = [(W^UK_h)^T q_nope[b][h] ; RoPE_pos(q_pe[b][h])]
__global__ __launch_bounds__(kThreads) void absorb_generic_kernel(
    int H, int dh, int dc, int dr, double base, bool bf, const void* __restrict__ q_nope,
    const void* __restrict__ q_pe, const int32_t* __restrict__ positions,
    const void* __restrict__ w_uk, void* __restrict__ q_abs) {
  extern __shared__ float qn[];  // [dh]
  const int b = blockIdx.x, h = blockIdx.y;
  const int64_t row = static_cast<int64_t>(b) * H + h;
  for (int d = threadIdx.x; d < dh; d += kThreads) qn[d] = load_elem(q_nope, row * dh + d, bf);
  __syncthreads();
  const int D = dc + dr;
  for (int c = threadIdx.x; c < dc; c += kThreads) {
    float acc = 0.f;
    for (int d = 0; d < dh; ++d)
      acc = fmaf(qn[d], load_elem(w_uk, (static_cast<int64_t>(h) * dh + d) * dc + c, bf), acc);
    store_elem(q_abs, row * D + c, acc, bf);
  }
  const double pos = static_cast<double>(positions[b]);
  for (int k = threadIdx.x; k < dr / 2; k += kThreads) {
    const double theta = pow(base, -2.0 * k / dr);
    double s, c;
    sincos(pos * theta, &s, &c);
    const float cf = static_cast<float>(c), sf = static_cast<float>(s);
    const float x0 = load_elem(q_pe, row * dr + 2 * k, bf);
    const float x1 = load_elem(q_pe, row * dr + 2 * k + 1, bf);
    store_elem(q_abs, row * D + dc + 2 * k, x0 * cf - x1 * sf, bf);
    store_elem(q_abs, row * D + dc + 2 * k + 1, x0 * sf + x1 * cf, bf);
  }
}

// One workgroup per (work item, query token, head): 256 tokens at a time,
// online softmax.  Query token t of q_len sees cache rows [0, L - q_len + t].
__global__ __launch_bounds__(kThreads) void decode_generic_kernel(
    int H, int dc, int dr, int P, int q_len, float scale, bool bf, const void* __restrict__ q_abs,
    const void* __restrict__ cache, const int32_t* __restrict__ block_table, int max_pages,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ items,
    float* __restrict__ o_part, float* __restrict__ lse_part) {
  extern __shared__ int64_t smem64[];
  const int D = dc + dr;
  int64_t* rowoff = smem64;                                      // [256] row offsets
  float* q = reinterpret_cast<float*>(rowoff + kThreads);        // [D]
  float* p = q + D;                                              // [256]
  float* red = p + kThreads;                                     // [8]
  const int it = blockIdx.x / q_len, tq = blockIdx.x % q_len, h = blockIdx.y;
  const int b = items[4 * it], p0 = items[4 * it + 2], p1 = items[4 * it + 3];
  const int L = seq_lens[b];
  const int t0 = p0 * P;
  const int t1 = min(p1 * P, L - q_len + tq + 1);
  const int64_t qrow = (static_cast<int64_t>(b) * q_len + tq) * H + h;
  const int64_t orow = (static_cast<int64_t>(it) * q_len + tq) * H + h;
  if (t1 <= t0) {  // the whole range lies after this token: an empty partial
    for (int c = threadIdx.x; c < dc; c += kThreads) o_part[orow * dc + c] = 0.f;
    if (threadIdx.x == 0) lse_part[orow] = -INFINITY;
    return;
  }
  for (int k = threadIdx.x; k < D; k += kThreads) q[k] = load_elem(q_abs, qrow * D + k, bf);
  constexpr int kMaxPer = 1024 / kThreads;  // d_c <= 1024
  float o[kMaxPer];
  for (int i = 0; i < kMaxPer; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  __syncthreads();
  for (int tb = t0; tb < t1; tb += kThreads) {
    const int t = tb + threadIdx.x;
    float s = -INFINITY;
    if (t < t1) {
      const int64_t page = block_table[static_cast<int64_t>(b) * max_pages + t / P];
      const int64_t off = (page * P + t % P) * D;
      rowoff[threadIdx.x] = off;
      float acc = 0.f;
      for (int k = 0; k < D; ++k) acc = fmaf(q[k], load_elem(cache, off + k, bf), acc);
      s = acc * scale;
    }
    const float mb = block_reduce_max(s, red);
    const float mn = fmaxf(m, mb);
    const float alpha = expf(m - mn);  // m = -inf on the first block: alpha = 0
    const float e = (t < t1) ? expf(s - mn) : 0.f;
    p[threadIdx.x] = e;
    const float sum = block_reduce_sum(e, red + 4);
    l = l * alpha + sum;
    m = mn;
    __syncthreads();
    const int n = min(kThreads, t1 - tb);
    for (int i = 0; i < kMaxPer; ++i) {
      const int c = threadIdx.x + i * kThreads;
      if (c >= dc) break;
      float acc = o[i] * alpha;
      for (int j = 0; j < n; ++j) acc = fmaf(p[j], load_elem(cache, rowoff[j] + c, bf), acc);
      o[i] = acc;
    }
    __syncthreads();
  }
  const float inv = 1.f / l;
  for (int i = 0; i < kMaxPer; ++i) {
    const int c = threadIdx.x + i * kThreads;
    if (c >= dc) break;
    o_part[orow * dc + c] = o[i] * inv;
  }
  if (threadIdx.x == 0) lse_part[orow] = m + logf(l);
}

__global__ __launch_bounds__(kThreads) void combine_generic_kernel(
    int H, int dc, int q_len, const int32_t* __restrict__ offs, const float* __restrict__ o_part,
    const float* __restrict__ lse_part, float* __restrict__ o_latent, float* __restrict__ lse) {
  // row r = b * q_len + t (query token t of sequence b); its partial in item s
  // is row s * q_len + t
  const int r = blockIdx.x, h = blockIdx.y;
  const int b = r / q_len, t = r % q_len;
  const int s0 = offs[b], s1 = offs[b + 1];
  auto prow = [&](int s) { return (static_cast<int64_t>(s) * q_len + t) * H + h; };
  float M = -INFINITY;
  for (int s = s0; s < s1; ++s) M = fmaxf(M, lse_part[prow(s)]);
  float Z = 0.f;
  for (int s = s0; s < s1; ++s) Z += expf(lse_part[prow(s)] - M);
  const float inv = 1.f / Z;
  for (int c = threadIdx.x; c < dc; c += kThreads) {
    float acc = 0.f;
    for (int s = s0; s < s1; ++s) acc = fmaf(expf(lse_part[prow(s)] - M), o_part[prow(s) * dc + c], acc);
    o_latent[(static_cast<int64_t>(r) * H + h) * dc + c] = acc * inv;
  }
  if (lse && threadIdx.x == 0) lse[static_cast<int64_t>(r) * H + h] = M + logf(Z);
}

// out[b][h][d] = sum_c W^UV[h*dh + d][c] * o_latent[b][h][c]; one wave per output row.
__global__ __launch_bounds__(kThreads) void out_proj_generic_kernel(
    int H, int dh, int dc, bool bf, const float* __restrict__ o_latent,
    const void* __restrict__ w_uv, float* __restrict__ out) {
  extern __shared__ float ol[];  // [dc]
  const int b = blockIdx.x, h = blockIdx.y;
  const int64_t row = static_cast<int64_t>(b) * H + h;
  for (int c = threadIdx.x; c < dc; c += kThreads) ol[c] = o_latent[row * dc + c];
  __syncthreads();
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  for (int d = w; d < dh; d += kThreads / 64) {
    float acc = 0.f;
    for (int c = l; c < dc; c += 64)
      acc = fmaf(load_elem(w_uv, (static_cast<int64_t>(h) * dh + d) * dc + c, bf), ol[c], acc);
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (l == 0) out[row * dh + d] = acc;
  }
}

}  // namespace

hipError_t absorb_generic(const mla_dims& d, int batch, const void* q_nope, const void* q_pe,
                          const int32_t* positions, const void* w_uk, void* q_abs,
                          hipStream_t stream) {
  const bool bf = d.dtype == MLA_BF16;
  hipLaunchKernelGGL(absorb_generic_kernel, dim3(batch, d.n_heads), dim3(kThreads),
                     d.d_head * sizeof(float), stream, d.n_heads, d.d_head, d.d_latent, d.d_rope,
                     d.rope_base, bf, q_nope, q_pe, positions, w_uk, q_abs);
  return hipGetLastError();
}

hipError_t decode_generic(const mla_dims& d, int q_len, const void* q_abs, const void* kv_cache,
                          const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                          const int32_t* items, int num_items, float* o_part, float* lse_part,
                          hipStream_t stream) {
  const bool bf = d.dtype == MLA_BF16;
  const size_t sm = (d.d_latent + d.d_rope + kThreads + 8) * sizeof(float) + kThreads * sizeof(int64_t);
  const int64_t blocks = static_cast<int64_t>(num_items) * q_len;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_generic_kernel, dim3(static_cast<uint32_t>(blocks), d.n_heads),
                     dim3(kThreads), sm, stream, d.n_heads, d.d_latent, d.d_rope, d.page_size, q_len,
                     d.softmax_scale, bf, q_abs,
                     kv_cache, block_table, max_pages, seq_lens, items, o_part, lse_part);
  return hipGetLastError();
}

hipError_t combine_generic(const mla_dims& d, int batch, int q_len, const int32_t* split_offsets,
                           const float* o_part, const float* lse_part, float* o_latent, float* lse,
                           hipStream_t stream) {
  hipLaunchKernelGGL(combine_generic_kernel, dim3(batch * q_len, d.n_heads), dim3(kThreads), 0, stream,
                     d.n_heads, d.d_latent, q_len, split_offsets, o_part, lse_part, o_latent, lse);
  return hipGetLastError();
}

hipError_t out_proj_generic(const mla_dims& d, int batch, const float* o_latent, const void* w_uv,
                            float* out, hipStream_t stream) {
  const bool bf = d.dtype == MLA_BF16;
  hipLaunchKernelGGL(out_proj_generic_kernel, dim3(batch, d.n_heads), dim3(kThreads),
                     d.d_latent * sizeof(float), stream, d.n_heads, d.d_head, d.d_latent, bf,
                     o_latent, w_uv, out);
  return hipGetLastError();
}

}  // namespace mla
