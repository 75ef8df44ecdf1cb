// The two per-head weight products around the latent attention, gfx950 fast
// path (bf16, d_h = 128, d_c = 512, d_h^R = 64).
//
//  absorb:   q~_{b,i} = (W^UK_i)^T q^C_{b,i}  and  RoPE_{p_b}(q^R_{b,i})
//            (page "DeepSeek V2 技术解析" 2.2.1.1: W^UK absorbed on the query
//            side; 2.2.2: decoupled RoPE query, rotation R_m)
//  out_proj: o_{b,i} = W^UV_i o~_{b,i}
//            (same page 2.2.1.1: W^UV absorbed on the output side; page
//            "DeepSeek-V2/V3：大模型的两张账" "第一张账": the latent-space result is
//            mapped out afterwards)
//
// Both are batched GEMMs with one [128 x 512] weight per head; each workgroup
// takes one head and up to 64 sequences (16 per wave) so that every weight is
// read from HBM once per 64 sequences.  MFMA v_mfma_f32_16x16x32_bf16.
#include <math.h>

#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kWRowBytes = kDc * 2;  // 1024 bytes per weight row

__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr)
               : "memory");
}

#define MLA_VMCNT0 ((7 << 4) | (15 << 8))

// ---------------------------------------------------------------------------
// absorb: q~^T[512 x b] = (W^UK_h)^T[512 x 128] . q^C^T[128 x b].
// W^UK_h (128 KiB) is staged in LDS, rows swizzled like the decode cache, and
// read transposed (ds_read_b64_tr_b16) as the A operand.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 1) void absorb_kernel(
    int batch, int H, double rope_base, const uint16_t* __restrict__ q_nope,
    const uint16_t* __restrict__ q_pe, const int32_t* __restrict__ positions,
    const char* __restrict__ w_uk, uint16_t* __restrict__ q_abs) {
  __shared__ __attribute__((aligned(1024))) char lds[kDh * kWRowBytes];
  const uint32_t lds_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, q = lane & 15;

  // stage W^UK_h: wave w copies rows 32w .. 32w+31, one row per instruction
  const char* wh = w_uk + static_cast<int64_t>(h) * kDh * kWRowBytes;
#pragma unroll 8
  for (int i = 0; i < 32; ++i) {
    const int row = 32 * w + i;
    const uint32_t off = row * kWRowBytes + 16 * (lane ^ swz(row));
    dma16(wh, off, lds_base + row * kWRowBytes);
  }

  // RoPE part, float64 angle, float32 rotation: (b, k) pairs of this batch group
  const int b0 = blockIdx.y * 64;
  const int nb = min(64, batch - b0);
  for (int e = threadIdx.x; e < nb * (kDr / 2); e += 256) {
    const int b = b0 + e / (kDr / 2), k = e % (kDr / 2);
    const double theta = pow(rope_base, -2.0 * k / kDr);
    double sd, cd;
    sincos(static_cast<double>(positions[b]) * theta, &sd, &cd);
    const float c = static_cast<float>(cd), s = static_cast<float>(sd);
    const int64_t r = static_cast<int64_t>(b) * H + h;
    const uint32_t xy = *reinterpret_cast<const uint32_t*>(q_pe + r * kDr + 2 * k);
    const float x0 = bf16_bits_to_f32(static_cast<uint16_t>(xy & 0xffffu));
    const float x1 = bf16_bits_to_f32(static_cast<uint16_t>(xy >> 16));
    const uint32_t o = static_cast<uint32_t>(f32_to_bf16_bits(x0 * c - x1 * s)) |
                       (static_cast<uint32_t>(f32_to_bf16_bits(x0 * s + x1 * c)) << 16);
    *reinterpret_cast<uint32_t*>(q_abs + r * kDq + kDc + 2 * k) = o;
  }

  // B operand: q^C of sequence b = b0 + 16w + q, values 32ks + 8g .. +8
  const int b = b0 + 16 * w + q;
  const bool bvalid = b < batch;
  bf16x8 qn[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (bvalid)
      qn[ks] = *reinterpret_cast<const bf16x8*>(q_nope + (static_cast<int64_t>(b) * H + h) * kDh +
                                                32 * ks + 8 * g);
    else
      qn[ks] = bf16x8{};
  }
  __builtin_amdgcn_s_waitcnt(MLA_VMCNT0);
  __syncthreads();
  if (16 * w >= nb) return;  // no sequence for this wave (no barrier follows)

  // A operand rows d = 32ks + 8g + s (+4), columns 16cb + 4(q%4): source-lane
  // role q -> row 8g + q/4 of the k block, column chunk 2cb + (q%4)/2.
  const int arow = 8 * g + (q >> 2);
  const int sw0 = swz(arow), sw1 = swz(arow + 4);
  uint16_t* qrow = q_abs + (static_cast<int64_t>(b) * H + h) * kDq + 4 * g;
#pragma unroll 4
  for (int cb = 0; cb < 32; ++cb) {
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int ch = 2 * cb + ((q & 3) >> 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int r0 = 32 * ks + arow;
      const uint32_t o0 = r0 * kWRowBytes + 16 * (ch ^ sw0) + 8 * (q & 1);
      const uint32_t o1 = (r0 + 4) * kWRowBytes + 16 * (ch ^ sw1) + 8 * (q & 1);
      const short4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) short4_t*)((__attribute__((address_space(3))) char*)lds + o0));
      const short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) short4_t*)((__attribute__((address_space(3))) char*)lds + o1));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qn[ks], acc, 0, 0, 0);
    }
    // lane holds q~[16cb + 4g + i] of sequence b
    if (bvalid) {
      const uint32_t lo = static_cast<uint32_t>(f32_to_bf16_bits(acc[0])) |
                          (static_cast<uint32_t>(f32_to_bf16_bits(acc[1])) << 16);
      const uint32_t hi = static_cast<uint32_t>(f32_to_bf16_bits(acc[2])) |
                          (static_cast<uint32_t>(f32_to_bf16_bits(acc[3])) << 16);
      uint32_t* dst = reinterpret_cast<uint32_t*>(qrow + 16 * cb);
      dst[0] = lo;
      dst[1] = hi;
    }
  }
}

// ---------------------------------------------------------------------------
// out_proj: o^T[128 x b] = W^UV_h[128 x 512] . o~^T[512 x b].  The float32 o~
// is split into bf16 hi + lo (lo = bf16(x - hi)); two MFMAs per step.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void out_proj_kernel(int batch, int H,
                                                       const float* __restrict__ o_lat,
                                                       const uint16_t* __restrict__ w_uv,
                                                       float* __restrict__ out) {
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4, q = lane & 15;
  const int bblk = blockIdx.y * 4 + w;
  if (bblk * 16 >= batch) return;
  const int b = bblk * 16 + q;
  const bool bvalid = b < batch;
  const float* orow = o_lat + (static_cast<int64_t>(b) * H + h) * kDc + 8 * g;
  const uint16_t* wrow = w_uv + (static_cast<int64_t>(h) * kDh + q) * kDc + 8 * g;
  float4_t acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int ks = 0; ks < 16; ++ks) {
    float x[8];
    if (bvalid) {
      const float4_t x0 = *reinterpret_cast<const float4_t*>(orow + 32 * ks);
      const float4_t x1 = *reinterpret_cast<const float4_t*>(orow + 32 * ks + 4);
      x[0] = x0[0]; x[1] = x0[1]; x[2] = x0[2]; x[3] = x0[3];
      x[4] = x1[0]; x[5] = x1[1]; x[6] = x1[2]; x[7] = x1[3];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.f;
    }
    uint16_t hb[8], lb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hb[j] = f32_to_bf16_bits(x[j]);
      lb[j] = f32_to_bf16_bits(x[j] - bf16_bits_to_f32(hb[j]));
    }
    const bf16x8 bhi = __builtin_bit_cast(bf16x8, hb);
    const bf16x8 blo = __builtin_bit_cast(bf16x8, lb);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(wrow + (16 * db) * kDc + 32 * ks);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bhi, acc[db], 0, 0, 0);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, blo, acc[db], 0, 0, 0);
    }
  }
  if (!bvalid) return;
  float* dst = out + (static_cast<int64_t>(b) * H + h) * kDh + 4 * g;
#pragma unroll
  for (int db = 0; db < 8; ++db) *reinterpret_cast<float4_t*>(dst + 16 * db) = acc[db];
}

}  // namespace

hipError_t absorb_fast(const mla_dims& d, int batch, const void* q_nope, const void* q_pe,
                       const int32_t* positions, const void* w_uk, void* q_abs,
                       hipStream_t stream) {
  const int groups = (batch + 63) / 64;
  if (groups > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(absorb_kernel, dim3(d.n_heads, groups), dim3(256), 0, stream, batch,
                     d.n_heads, d.rope_base, static_cast<const uint16_t*>(q_nope),
                     static_cast<const uint16_t*>(q_pe), positions,
                     static_cast<const char*>(w_uk), static_cast<uint16_t*>(q_abs));
  return hipGetLastError();
}

hipError_t out_proj_fast(const mla_dims& d, int batch, const float* o_latent, const void* w_uv,
                         float* out, hipStream_t stream) {
  const int groups = (batch + 63) / 64;
  if (groups > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(out_proj_kernel, dim3(d.n_heads, groups), dim3(256), 0, stream, batch,
                     d.n_heads, o_latent, static_cast<const uint16_t*>(w_uv), out);
  return hipGetLastError();
}

}  // namespace mla
