// Log-sum-exp merge of the split-KV partials, d_c = 512.
//
// One workgroup of 128 threads per (sequence, head): every thread owns four
// consecutive latent columns (one 16-byte float4 per partial).  Softmax over a
// union of disjoint token sets: with M = max_s lse_s and w_s = exp(lse_s - M),
// o = sum_s w_s o_s / sum_s w_s and lse = M + log sum_s w_s.
#include <math.h>

#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

__global__ __launch_bounds__(128) void combine_512_kernel(
    int H, int q_len, const int32_t* __restrict__ offs, const float* __restrict__ o_part,
    const float* __restrict__ lse_part, float* __restrict__ o_latent, float* __restrict__ lse) {
  // row rr = b * q_len + t (query token t of sequence b); its partial in item
  // s is row s * q_len + t
  const int rr = blockIdx.x / H, h = blockIdx.x % H;
  const int b = rr / q_len, t = rr % q_len;
  const int s0 = offs[b], s1 = offs[b + 1];
  float M = -INFINITY;
  for (int s = s0; s < s1; ++s) M = fmaxf(M, lse_part[(static_cast<int64_t>(s) * q_len + t) * H + h]);
  float Z = 0.f;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = s0; s < s1; ++s) {
    const int64_t r = (static_cast<int64_t>(s) * q_len + t) * H + h;
    const float w = expf(lse_part[r] - M);
    Z += w;
    const float4_t v = reinterpret_cast<const float4_t*>(o_part + r * kDc)[threadIdx.x];
    acc[0] = fmaf(w, v[0], acc[0]);
    acc[1] = fmaf(w, v[1], acc[1]);
    acc[2] = fmaf(w, v[2], acc[2]);
    acc[3] = fmaf(w, v[3], acc[3]);
  }
  const float inv = 1.f / Z;
  acc[0] *= inv;
  acc[1] *= inv;
  acc[2] *= inv;
  acc[3] *= inv;
  const int64_t ro = static_cast<int64_t>(rr) * H + h;
  reinterpret_cast<float4_t*>(o_latent + ro * kDc)[threadIdx.x] = acc;
  if (lse && threadIdx.x == 0) lse[ro] = M + logf(Z);
}

}  // namespace

hipError_t combine_fast(const mla_dims& d, int batch, int q_len, const int32_t* split_offsets,
                        const float* o_part, const float* lse_part, float* o_latent, float* lse,
                        hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(batch) * q_len * d.n_heads;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_512_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(128), 0, stream,
                     d.n_heads, q_len, split_offsets, o_part, lse_part, o_latent, lse);
  return hipGetLastError();
}

}  // namespace mla
