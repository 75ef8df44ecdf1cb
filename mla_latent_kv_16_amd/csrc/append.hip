// Cache write of the decoded token (one per sequence): the row that the decode
// step reads back from the paged latent cache.
//
// Page "DeepSeek V2 技术解析" 2.2.1.1 (the joint latent c^KV = W^DKV h_t is all
// that is kept of the keys and values) and 2.2.2 (the decoupled key
// k^R_t = W^KR h_t is shared by the heads and cached after the rotation R_t);
// page "DeepSeek-V2/V3：大模型的两张账", "第一张账" (the cached latent is
// normalised).  For every sequence b with hidden state h_b at position p_b:
//   c_b  = W^DKV h_b, then c_b / sqrt(mean(c_b^2) + eps) when rms_norm is set
//   kr_b = RoPE_{p_b}(W^KR h_b)       (angles p_b theta_k in float64)
//   cache row (page block_table[b][p_b / page], slot p_b % page) = [c_b | kr_b]
//
// Two launches:
//  * project: the [batch x d_model] . [d_model x (d_c + d_h^R)] products in
//    K-slices, float32 partial sums into the caller's workspace.  On the bf16
//    fast path each wave computes one 16 x 16 tile of one K-slice with
//    v_mfma_f32_16x16x32_bf16, both operands read straight from global memory
//    (h and the weight rows are contiguous along d_model, the reduction).
//  * finish: per sequence, the K-slices summed in order (deterministic), the
//    RMS norm over the latent, the rotation, the rounding to the storage type
//    and the scatter into the cache slot.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kKSlice = 640;  // d_model values per K-slice (20 MFMA steps)
constexpr int kSteps = kKSlice / 32;

__global__ __launch_bounds__(64) void append_project_mfma(
    int batch, int d_model, int D, const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_dkv,
    const uint16_t* __restrict__ w_kr, int dc, float* __restrict__ ws) {
  const int lane = threadIdx.x, g = lane >> 4, q = lane & 15;
  const int cb = blockIdx.x, bb = blockIdx.y, ks0 = blockIdx.z * kKSlice;
  const int col = 16 * cb + q;  // output column of this lane's B operand row
  const uint16_t* wrow = col < dc ? w_dkv + static_cast<int64_t>(col) * d_model
                                  : w_kr + static_cast<int64_t>(col - dc) * d_model;
  const int b = 16 * bb + q;
  const bool bvalid = b < batch;
  const uint16_t* hrow = h + static_cast<int64_t>(bvalid ? b : 0) * d_model;
  const int kend = min(d_model, ks0 + kKSlice);
  // Every load of the slice is issued before the first MFMA, so the wave waits
  // for memory once instead of once per step.  Steps past d_model (the last
  // slice may be short; d_model % 32 == 0) load the slice's first step again,
  // a valid address, and are dropped below.
  bf16x8 av[kSteps], wv[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int kk = ks0 + 32 * i;
    const int k = (kk < kend ? kk : ks0) + 8 * g;
    av[i] = *reinterpret_cast<const bf16x8*>(hrow + k);
    wv[i] = *reinterpret_cast<const bf16x8*>(wrow + k);
  }
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    if (ks0 + 32 * i < kend) {  // uniform
      const bf16x8 a = bvalid ? av[i] : bf16x8{};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, wv[i], acc, 0, 0, 0);
    }
  }
  // lane holds D[b = 16bb + 4g + i][col = 16cb + q]
  float* out = ws + (static_cast<int64_t>(blockIdx.z) * batch) * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bi = 16 * bb + 4 * g + i;
    if (bi < batch) out[static_cast<int64_t>(bi) * D + col] = acc[i];
  }
}

// any shape / storage type: one thread per (sequence, output column, K-slice)
__global__ __launch_bounds__(256) void append_project_generic(
    int batch, int d_model, int D, bool bf, const void* __restrict__ h, const void* __restrict__ w_dkv,
    const void* __restrict__ w_kr, int dc, float* __restrict__ ws) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int b = blockIdx.y, s = blockIdx.z;
  if (t >= D) return;
  const int col = static_cast<int>(t);
  const int ks0 = s * kKSlice, kend = min(d_model, ks0 + kKSlice);
  float acc = 0.f;
  for (int k = ks0; k < kend; ++k) {
    const float x = load_elem(h, static_cast<int64_t>(b) * d_model + k, bf);
    const float wv = col < dc ? load_elem(w_dkv, static_cast<int64_t>(col) * d_model + k, bf)
                              : load_elem(w_kr, static_cast<int64_t>(col - dc) * d_model + k, bf);
    acc = fmaf(x, wv, acc);
  }
  ws[(static_cast<int64_t>(s) * batch + b) * D + col] = acc;
}

__global__ __launch_bounds__(1024) void append_finish(
    int batch, int dc, int dr, int n_slices, bool bf, bool rms_norm, float eps, double rope_base,
    const int32_t* __restrict__ positions, const float* __restrict__ ws, void* __restrict__ cache,
    int page_size, const int32_t* __restrict__ block_table, int max_pages) {
  extern __shared__ float row[];  // [dc + dr], then one float per wave for the reduction
  const int b = blockIdx.x;
  const int D = dc + dr;
  float* red = row + D;
  float ss = 0.f;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    // the slices in order, eight loads in flight at a time
    float v = 0.f;
    int s = 0;
    for (; s + 8 <= n_slices; s += 8) {
      float t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = ws[(static_cast<int64_t>(s + j) * batch + b) * D + c];
#pragma unroll
      for (int j = 0; j < 8; ++j) v += t[j];
    }
    for (; s < n_slices; ++s) v += ws[(static_cast<int64_t>(s) * batch + b) * D + c];
    row[c] = v;
    if (c < dc) ss = fmaf(v, v, ss);
  }
  // sum of squares of the latent over the workgroup
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float scale = 1.f;
  if (rms_norm) {
    float tot = 0.f;
    for (int i = 0; i < static_cast<int>(blockDim.x >> 6); ++i) tot += red[i];
    scale = 1.f / sqrtf(tot / static_cast<float>(dc) + eps);
  }
  const int pos = positions[b];
  const int page = block_table[static_cast<int64_t>(b) * max_pages + pos / page_size];
  const int64_t base = (static_cast<int64_t>(page) * page_size + pos % page_size) * D;
  for (int c = threadIdx.x; c < dc; c += blockDim.x) store_elem(cache, base + c, row[c] * scale, bf);
  for (int k = threadIdx.x; k < dr / 2; k += blockDim.x) {
    const double theta = pow(rope_base, -2.0 * k / dr);
    double sd, cd;
    sincos(static_cast<double>(pos) * theta, &sd, &cd);
    const float cs = static_cast<float>(cd), sn = static_cast<float>(sd);
    const float x0 = row[dc + 2 * k], x1 = row[dc + 2 * k + 1];
    store_elem(cache, base + dc + 2 * k, x0 * cs - x1 * sn, bf);
    store_elem(cache, base + dc + 2 * k + 1, x0 * sn + x1 * cs, bf);
  }
}

// Scratch of mla_append_kv_noalloc: the K-slice partial sums live in this
// static array instead of a caller's workspace.  Every device the library
// runs on holds its own copy until the process ends.  In host code `scratch`
// is only a stand-in for the symbol: its device address on the current device
// comes from hipGetSymbolAddress (scratch_on_current_device).
static __device__ __align__(256) float scratch[kAppendScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_on_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<float*>(g_scratch_ptr[dev]);
  return hipSuccess;
}

int append_slices(int d_model) { return (d_model + kKSlice - 1) / kKSlice; }

hipError_t append_kv(const mla_dims& d, int d_model, int batch, const void* h, const void* w_dkv,
                     const void* w_kr, const int32_t* positions, bool rms_norm, float eps,
                     void* kv_cache, const int32_t* block_table, int max_pages, float* ws,
                     hipStream_t stream) {
  const int D = d.d_latent + d.d_rope;
  const int S = append_slices(d_model);
  const bool bf = d.dtype == MLA_BF16;
  if (bf && d_model % 32 == 0 && D % 16 == 0 && d.d_latent % 16 == 0) {
    hipLaunchKernelGGL(append_project_mfma, dim3(D / 16, (batch + 15) / 16, S), dim3(64), 0, stream,
                       batch, d_model, D, static_cast<const uint16_t*>(h),
                       static_cast<const uint16_t*>(w_dkv), static_cast<const uint16_t*>(w_kr),
                       d.d_latent, ws);
  } else {
    hipLaunchKernelGGL(append_project_generic, dim3((D + 255) / 256, batch, S), dim3(256), 0, stream,
                       batch, d_model, D, bf, h, w_dkv, w_kr, d.d_latent, ws);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one thread per output column where D allows (up to 1024), so each thread's
  // slice loads are all in flight at once
  const int threads = std::min(1024, (D + 63) / 64 * 64);
  hipLaunchKernelGGL(append_finish, dim3(batch), dim3(threads), (D + threads / 64) * sizeof(float),
                     stream, batch,
                     d.d_latent, d.d_rope, S, bf, rms_norm, eps, d.rope_base, positions, ws, kv_cache,
                     d.page_size, block_table, max_pages);
  return hipGetLastError();
}

}  // namespace mla
