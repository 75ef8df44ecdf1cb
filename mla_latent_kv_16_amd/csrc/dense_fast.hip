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


__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr)
               : "memory");
}

#define MLA_VMCNT0 ((7 << 4) | (15 << 8))

// XCD-aware workgroup numbering: workgroup i runs on XCD i % 8.  Give the
// `per` consecutive blocks of one head the same XCD so they share its L2.
__device__ __forceinline__ void xcd_split(int i, int per, int& head, int& sub) {
  const int xcd = i & 7, k = i >> 3;
  sub = k % per;
  head = (k / per) * 8 + xcd;
}

// ---------------------------------------------------------------------------
// absorb: q~^T[512 x b] = (W^UK_h)^T[512 x 128] . q^C^T[128 x b], one
// workgroup per (head, quarter of the 512 latent columns, 64 sequences).
// The [128 x 128] weight tile (32 KiB) is staged in LDS, rows of 256 bytes with
// chunk position ch ^ tsw(row), and read transposed (ds_read_b64_tr_b16) as
// the A operand: each half-wave then touches rows {r..r+3, r+8..r+11} x two
// adjacent chunks, 16 distinct 16-byte bank groups.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tsw(int row) { return ((row & 3) << 1) | (((row >> 3) & 1) << 3); }

__global__ __launch_bounds__(256) void absorb_kernel(
    int batch, int H, double rope_base, const uint16_t* __restrict__ q_nope,
    const uint16_t* __restrict__ q_pe, const int32_t* __restrict__ positions,
    const char* __restrict__ w_uk, uint16_t* __restrict__ q_abs) {
  constexpr int kCols = 128, kTileRow = kCols * 2;  // 256 bytes
  __shared__ __attribute__((aligned(1024))) char lds[kDh * kTileRow];
  const uint32_t lds_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));
  int h, quarter;
  xcd_split(blockIdx.x, 4, h, quarter);
  const int c0 = quarter * kCols;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, q = lane & 15;

  // stage W^UK_h[:, c0:c0+128]: LDS chunk p = row * 16 + pc holds chunk pc ^ tsw(row)
  const char* wh = w_uk + static_cast<int64_t>(h) * kDh * (kDc * 2) + c0 * 2;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = (8 * w + i) * 64 + lane;
    const int row = p >> 4, pc = p & 15;
    dma16(wh, row * (kDc * 2) + 16 * (pc ^ tsw(row)), lds_base + (8 * w + i) * 1024);
  }

  const int b0 = blockIdx.y * 64;
  const int nb = min(64, batch - b0);
  // RoPE part, float64 angle, float32 rotation.  The four quarter-workgroups
  // of a head share the (sequence, pair) list; thread t keeps pair k = t % 32.
  {
    const int k = threadIdx.x & (kDr / 2 - 1);
    const double theta = pow(rope_base, -2.0 * k / kDr);
    for (int bi = quarter * 8 + (threadIdx.x >> 5); bi < nb; bi += 32) {
      const int bb = b0 + bi;
      double sd, cd;
      sincos(static_cast<double>(positions[bb]) * theta, &sd, &cd);
      const float c = static_cast<float>(cd), sn = static_cast<float>(sd);
      const int64_t r = static_cast<int64_t>(bb) * H + h;
      const uint32_t xy = *reinterpret_cast<const uint32_t*>(q_pe + r * kDr + 2 * k);
      const float x0 = bf16_bits_to_f32(static_cast<uint16_t>(xy & 0xffffu));
      const float x1 = bf16_bits_to_f32(static_cast<uint16_t>(xy >> 16));
      *reinterpret_cast<uint32_t*>(q_abs + r * kDq + kDc + 2 * k) =
          pack_bf16x2(x0 * c - x1 * sn, x0 * sn + x1 * c);
    }
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

  // A operand rows d = 32ks + 8g + s (+4), columns 16cb + 4(q%4) of the tile:
  // source-lane role q -> row 8g + q/4 of the k block, chunk 2cb + (q%4)/2.
  const int arow = 8 * g + (q >> 2);
  const int sw0 = tsw(arow), sw1 = tsw(arow + 4);
  uint16_t* qrow = q_abs + (static_cast<int64_t>(b) * H + h) * kDq + c0 + 4 * g;
#pragma unroll
  for (int cb = 0; cb < kCols / 16; ++cb) {
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int ch = 2 * cb + ((q & 3) >> 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int r0 = 32 * ks + arow;
      const uint32_t o0 = r0 * kTileRow + 16 * (ch ^ sw0) + 8 * (q & 1);
      const uint32_t o1 = (r0 + 4) * kTileRow + 16 * (ch ^ sw1) + 8 * (q & 1);
      const short4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) short4_t*)((__attribute__((address_space(3))) char*)lds + o0));
      const short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) short4_t*)((__attribute__((address_space(3))) char*)lds + o1));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qn[ks], acc, 0, 0, 0);
    }
    // lane holds q~[c0 + 16cb + 4g + i] of sequence b
    if (bvalid) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(qrow + 16 * cb);
      dst[0] = pack_bf16x2(acc[0], acc[1]);
      dst[1] = pack_bf16x2(acc[2], acc[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// out_proj: o^T[64 x b] = W^UV_h[64 rows x 512] . o~^T[512 x b], one workgroup
// per (head, half of the 128 output rows, 64 sequences); the two halves of a
// head run on one XCD and share its o~ through the L2.  The float32 o~ of the
// 64 sequences is staged once in LDS as bf16 hi + lo (lo = bf16(x - hi)),
// rows of 1 KiB with 16-byte chunk c at position c ^ 2 (b % 8): the B-operand
// reads (16 sequences x one chunk per quarter-wave) then hit distinct bank
// groups.  Wave w owns output rows 16w .. 16w+15 of the half for all 64
// sequences (four accumulators), W^UV rows straight from global memory.
// ---------------------------------------------------------------------------
constexpr int kOutSeq = 64;
constexpr int kOutHalfBytes = kOutSeq * kDc * 2;  // one bf16 copy of the staged o~

__global__ __launch_bounds__(256) void out_proj_kernel(int batch, int H,
                                                       const float* __restrict__ o_lat,
                                                       const uint16_t* __restrict__ w_uv,
                                                       float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kOutHalfBytes];  // [hi | lo][b][512]
  int h, half;
  xcd_split(blockIdx.x, 2, h, half);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, q = lane & 15;
  const int b0 = blockIdx.y * kOutSeq;
  const int nb = min(kOutSeq, batch - b0);

  // A operand: W^UV row 64 half + 16w + q, values 32ks + 8g .. +8
  const int drow = 64 * half + 16 * w + q;
  const uint16_t* wrow = w_uv + (static_cast<int64_t>(h) * kDh + drow) * kDc + 8 * g;
  bf16x8 a[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) a[ks] = *reinterpret_cast<const bf16x8*>(wrow + 32 * ks);

  // stage o~: float4 f = t + 256 i covers sequence f / 128, values 4 (f % 128) .. +4
#pragma unroll
  for (int i0 = 0; i0 < 32; i0 += 8) {
    float4_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int f = threadIdx.x + 256 * (i0 + i);
      const int bl = f >> 7;
      v[i] = bl < nb ? *reinterpret_cast<const float4_t*>(
                           o_lat + (static_cast<int64_t>(b0 + bl) * H + h) * kDc + 4 * (f & 127))
                     : float4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int f = threadIdx.x + 256 * (i0 + i);
      const int bl = f >> 7, c = 4 * (f & 127);
      const uint32_t off = bl * (kDc * 2) + 16 * ((c >> 3) ^ (2 * (bl & 7))) + 2 * (c & 7);
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        hi[j] = pack_bf16x2(v[i][2 * j], v[i][2 * j + 1]);
        lo[j] = pack_bf16x2(v[i][2 * j] - __uint_as_float(hi[j] << 16),
                            v[i][2 * j + 1] - __uint_as_float(hi[j] & 0xffff0000u));
      }
      *reinterpret_cast<uint64_t*>(lds + off) = (static_cast<uint64_t>(hi[1]) << 32) | hi[0];
      *reinterpret_cast<uint64_t*>(lds + kOutHalfBytes + off) = (static_cast<uint64_t>(lo[1]) << 32) | lo[0];
    }
  }
  __syncthreads();

  // B operand: sequence 16bb + q, values 32ks + 8g .. +8 (chunk 4ks + g)
  float4_t acc[4] = {};
  const uint32_t brow = q * (kDc * 2);
  const int bsw = 2 * (q & 7);
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const uint32_t col = 16 * ((4 * ks + g) ^ bsw);
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const uint32_t off = bb * 16 * (kDc * 2) + brow + col;
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(lds + off);
      const bf16x8 bl = *reinterpret_cast<const bf16x8*>(lds + kOutHalfBytes + off);
      acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], bh, acc[bb], 0, 0, 0);
      acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], bl, acc[bb], 0, 0, 0);
    }
  }
  // lane holds o[b0 + 16bb + q][h][64 half + 16w + 4g + i]
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const int bl = 16 * bb + q;
    if (bl < nb)
      *reinterpret_cast<float4_t*>(out + (static_cast<int64_t>(b0 + bl) * H + h) * kDh + 64 * half +
                                   16 * w + 4 * g) = acc[bb];
  }
}

}  // namespace

hipError_t absorb_fast(const mla_dims& d, int batch, const void* q_nope, const void* q_pe,
                       const int32_t* positions, const void* w_uk, void* q_abs,
                       hipStream_t stream) {
  const int groups = (batch + 63) / 64;
  if (groups > 65535 || d.n_heads % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(absorb_kernel, dim3(d.n_heads * 4, groups), dim3(256), 0, stream, batch,
                     d.n_heads, d.rope_base, static_cast<const uint16_t*>(q_nope),
                     static_cast<const uint16_t*>(q_pe), positions,
                     static_cast<const char*>(w_uk), static_cast<uint16_t*>(q_abs));
  return hipGetLastError();
}

hipError_t out_proj_fast(const mla_dims& d, int batch, const float* o_latent, const void* w_uv,
                         float* out, hipStream_t stream) {
  const int groups = (batch + 63) / 64;
  if (groups > 65535 || d.n_heads % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(out_proj_kernel, dim3(d.n_heads * 2, groups), dim3(256), 0, stream, batch,
                     d.n_heads, o_latent, static_cast<const uint16_t*>(w_uv), out);
  return hipGetLastError();
}

}  // namespace mla
