// Prefill through the naive, materialised-K/V path: the q_len newest tokens
// of each sequence (all already in the cache) attend causally to the cache,
// with the per-head keys and values recovered from the latent first.
//
// Page "DeepSeek V2 技术解析" 2.2.1.1 (k^C = W^UK c^KV and v^C = W^UV c^KV: the
// up-projections recover per-head keys and values from the joint latent), 2.2.1.2
// (a query sees only the tokens up to its own) and 2.2.2 (the key is
// [k^C ; RoPE(k^R)] with one k^R shared by all heads, the query [q^C ; RoPE(q^R)]).
// For sequence b of length L, head i and query token t at position p = L - q_len + t:
//   K_j = [W^UK_i c_j ; kr_j],  V_j = W^UV_i c_j          (j < L; kr_j is cached rotated)
//   q   = [q^C ; RoPE_p(q^R)]
//   o   = sum_{j <= p} softmax_j(scale * q . K_j) V_j,  lse = log sum_{j <= p} exp(scale * q . K_j)
//
// Two launches:
//  * materialise: K^C and V^C of every cached row, [b][i][j][128] bf16 each, in
//    the caller's workspace.  One workgroup of eight waves per (head, K or V,
//    sequence) holds W_i (128 KiB) in LDS and walks the sequence's rows, 16 per
//    wave at a time: D^T[128 x 16 rows] = W_i[128 x 512] . c^T[512 x 16 rows]
//    with v_mfma_f32_16x16x32_bf16, the latent rows read straight from the
//    paged cache, float32 accumulation rounded to bf16.
//  * attention: one workgroup of four waves per (128 query tokens, head,
//    sequence), one wave per 32 queries (two blocks of 16, so that every K or
//    V fragment read from LDS feeds two MFMAs); keys in tiles of 32 staged in
//    LDS for all four waves (K row-major, V transposed), with an online
//    softmax in base 2 whose reference moves only when the running maximum
//    gains more than 2^8 (the accumulators are rescaled only then).
//    S^T[16 keys x 16 queries] on MFMA (K rows as A, the query tile as B, 6
//    steps over the 192 dimensions), then O^T[128 x 16 queries] += V^T . P^T
//    with the reduction index running over the keys each lane's score
//    accumulators hold, so P^T needs no reshuffle.
#include <math.h>

#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr float kRefSlack = 8.f;   // log2 units the softmax reference may trail the running maximum
constexpr int kQB = 2;             // 16-query blocks per attention wave
constexpr int kQWave = 16 * kQB;   // query tokens per attention wave
constexpr int kKeyTile = 32;   // keys per attention iteration
constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;

struct PrefillTheta {
  double t[kDr / 2];  // theta_k = rope_base^(-2k / d_h^R), from the host in float64
};

// sin and cos of a float64 angle: reduced to [-pi, pi] in float64 (two-term
// Cody-Waite with fused multiply-adds), then sin/cos in float32
__device__ __forceinline__ void sincos_reduced(double x, float& sn, float& cs) {
  constexpr double kTwoPiHi = 6.283185307179586, kTwoPiLo = 2.4492935982947064e-16;
  const double n = rint(x * (1.0 / kTwoPiHi));
  double r = fma(-n, kTwoPiHi, x);
  r = fma(-n, kTwoPiLo, r);
  sincosf(static_cast<float>(r), &sn, &cs);
}

// Maximum / sum over the four lanes q, q+16, q+32, q+48 of a wave.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Row j of sequence b in the paged cache (the caller guarantees j < L_b).
__device__ __forceinline__ const uint16_t* cache_row(const uint16_t* cache, const int32_t* bt, int j) {
  return cache + (static_cast<int64_t>(bt[j >> 6]) * kPage + (j & (kPage - 1))) * kDq;
}

__global__ __launch_bounds__(512) void materialise_kv_kernel(
    int H, int max_rows, const uint16_t* __restrict__ cache, const int32_t* __restrict__ block_table,
    int max_pages, const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ w_uk,
    const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc) {
  // W_h (128 rows x 512, 128 KiB) in LDS, row r's 16-byte chunk c at position
  // c ^ (r % 16): the A-operand reads (16 rows x one chunk per quarter-wave)
  // then touch 16 distinct bank groups
  __shared__ __attribute__((aligned(16))) char wl[kDh * kDc * 2];
  const int h = blockIdx.x, which = blockIdx.y, b = blockIdx.z;
  const int L = seq_lens[b];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, q = lane & 15;
  const uint16_t* wh = (which ? w_uv : w_uk) + static_cast<int64_t>(h) * kDh * kDc;
  for (int idx = threadIdx.x; idx < kDh * (kDc / 8); idx += blockDim.x) {
    const int r = idx >> 6, c = idx & 63;
    *reinterpret_cast<bf16x8*>(wl + r * (kDc * 2) + 16 * (c ^ (r & 15))) =
        *reinterpret_cast<const bf16x8*>(wh + r * kDc + 8 * c);
  }
  __syncthreads();
  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_pages;
  uint16_t* dst0 = (which ? vc : kc) + (static_cast<int64_t>(b) * H + h) * max_rows * kDh;
  // wave w takes rows j0 + 16w .. +15 of every 128-row tile
  for (int j0 = 0; j0 < L; j0 += 8 * 16) {
    const int jb = j0 + 16 * w;
    if (jb >= L) continue;  // no barrier follows
    const int j = jb + q;   // this lane's row (B operand column)
    const bool jvalid = j < L;
    const uint16_t* crow = cache_row(cache, bt, jvalid ? j : jb) + 8 * g;
    bf16x8 cf[kDc / 32];
#pragma unroll
    for (int ks = 0; ks < kDc / 32; ++ks) cf[ks] = *reinterpret_cast<const bf16x8*>(crow + 32 * ks);
    uint16_t* dst = dst0 + static_cast<int64_t>(j) * kDh;
#pragma unroll
    for (int nb = 0; nb < kDh / 16; ++nb) {
      // A operand: W_h row 16nb + q, latent values 32ks + 8g .. +8 (chunk 4ks + g)
      const char* arow = wl + (16 * nb + q) * (kDc * 2);
      float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kDc / 32; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            *reinterpret_cast<const bf16x8*>(arow + 16 * ((4 * ks + g) ^ q)), cf[ks], acc, 0, 0, 0);
      // lane holds D^T[16nb + 4g + i][row j]
      if (jvalid) {
        const uint32_t lo = pack_bf16x2(acc[0], acc[1]), hi = pack_bf16x2(acc[2], acc[3]);
        *reinterpret_cast<uint64_t*>(dst + 16 * nb + 4 * g) = (static_cast<uint64_t>(hi) << 32) | lo;
      }
    }
  }
}

// K tile: 32 keys x 192 dimensions, rows padded to 400 bytes.  V tile: 32 keys
// x 128 dimensions, rows padded to 288 bytes, read transposed with
// ds_read_b64_tr_b16 (a 16-lane group reads 4 keys x 16 dimensions and each
// lane receives the 4 keys of one dimension; the 32-byte row shift puts the 8
// rows a half-wave reads in distinct bank groups).
constexpr int kKRowB = 2 * (kDh + kDr) + 16;  // 400
constexpr int kVRowB = 2 * kDh + 32;          // 288
constexpr int kAttnWaves = 4;                  // query tiles per workgroup

__device__ __forceinline__ uint64_t lds_tr4(const char* lds, uint32_t off) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)((__attribute__((address_space(3))) const char*)lds + off));
  return __builtin_bit_cast(uint64_t, v);
}

__global__ __launch_bounds__(64 * kAttnWaves, 2) void prefill_attn_kernel(
    int H, int q_len, int max_rows, float scale, PrefillTheta theta,
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const uint16_t* __restrict__ cache, const int32_t* __restrict__ block_table, int max_pages,
    const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) char ks_lds[kKeyTile * kKRowB];
  __shared__ __attribute__((aligned(16))) char v_lds[kKeyTile * kVRowB];
  const int b = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, q = lane & 15;
  const int L = seq_lens[b];
  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_pages;
  const int t0 = (blockIdx.x * kAttnWaves + w) * kQWave;   // this wave's first query
  // query block qb: tokens t0 + 16qb .. +15; this lane's token (B operand column)
  int pos[kQB];
  bool tvalid[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int t = t0 + 16 * qb + q;
    tvalid[qb] = t < q_len;
    pos[qb] = L - q_len + (tvalid[qb] ? t : q_len - 1);
  }
  // last position of this wave's and of the workgroup's queries (-1: none)
  const int p_wave = t0 < q_len ? L - q_len + min(t0 + kQWave, q_len) - 1 : -1;
  const int tw_end = min((blockIdx.x + 1) * kAttnWaves * kQWave, q_len);
  const int p_wg = L - q_len + tw_end - 1;

  // Query tiles as the B operand: dimensions 32ks + 8g .. +8 of the lane's token
  bf16x8 qf[kQB][6];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int t = t0 + 16 * qb + q;
    const int64_t row = (static_cast<int64_t>(b) * q_len + (tvalid[qb] ? t : 0)) * H + h;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[qb][ks] = *reinterpret_cast<const bf16x8*>(q_nope + row * kDh + 32 * ks + 8 * g);
#pragma unroll
    for (int ks = 4; ks < 6; ++ks) {
      const int d0 = 32 * (ks - 4) + 8 * g;  // rope dimensions d0 .. d0+7: pairs d0/2 .. d0/2+3
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(q_pe + row * kDr + d0);
      uint32_t pk[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float sn, cs;
        sincos_reduced(static_cast<double>(pos[qb]) * theta.t[d0 / 2 + m], sn, cs);
        const float x0 = static_cast<float>(x[2 * m]), x1 = static_cast<float>(x[2 * m + 1]);
        pk[m] = pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
      }
      qf[qb][ks] = __builtin_bit_cast(bf16x8, pk);
    }
  }

  const float c2 = scale * kLog2eF;
  const uint16_t* kh = kc + (static_cast<int64_t>(b) * H + h) * max_rows * kDh;
  const uint16_t* vh = vc + (static_cast<int64_t>(b) * H + h) * max_rows * kDh;
  float4_t o[kQB][kDh / 16];
  float m_run[kQB], l_run[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
    for (int db = 0; db < kDh / 16; ++db) o[qb][db] = float4_t{0.f, 0.f, 0.f, 0.f};
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  // Tile staging, software-pipelined: the 256 threads load the next tile into
  // registers (K^C and V: keys i/16 and 16 + i/16, chunk i%16; k^R: key i/8,
  // chunk i%8) while the waves compute on the one in LDS.
  static_assert(kKeyTile * 16 == 2 * 64 * kAttnWaves && kKeyTile * 8 == 64 * kAttnWaves, "staging split");
  bf16x8 rk[2], rv[2], rr;
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + u * 64 * kAttnWaves;
      const int key = min(k0 + (i >> 4), L - 1);
      rk[u] = *reinterpret_cast<const bf16x8*>(kh + static_cast<int64_t>(key) * kDh + 8 * (i & 15));
      rv[u] = *reinterpret_cast<const bf16x8*>(vh + static_cast<int64_t>(key) * kDh + 8 * (i & 15));
    }
    const int key = min(k0 + (threadIdx.x >> 3), L - 1);
    rr = *reinterpret_cast<const bf16x8*>(cache_row(cache, bt, key) + kDc + 8 * (threadIdx.x & 7));
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + u * 64 * kAttnWaves;
      *reinterpret_cast<bf16x8*>(ks_lds + (i >> 4) * kKRowB + 16 * (i & 15)) = rk[u];
      *reinterpret_cast<bf16x8*>(v_lds + (i >> 4) * kVRowB + 16 * (i & 15)) = rv[u];
    }
    *reinterpret_cast<bf16x8*>(ks_lds + (threadIdx.x >> 3) * kKRowB + 2 * kDh + 16 * (threadIdx.x & 7)) = rr;
  };
  load_tile(0);
  for (int k0 = 0; k0 <= p_wg; k0 += kKeyTile) {
    __syncthreads();  // the previous tile is no longer read
    store_tile();
    if (k0 + kKeyTile <= p_wg) load_tile(k0 + kKeyTile);
    __syncthreads();
    if (k0 > p_wave) continue;  // every key of the tile lies after this wave's queries

    // S^T for keys k0 + 16kb + row, queries of block qb: lane holds keys
    // 16kb + 4g + i.  Each row fragment read from LDS feeds one MFMA per
    // query block.
    float s[kQB][2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const char* krow = ks_lds + (16 * kb + q) * kKRowB + 16 * g;
      float4_t acc[kQB];
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) acc[qb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 64 * ks);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          acc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][ks], acc[qb], 0, 0, 0);
      }
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + 16 * kb + 4 * g + i;
          s[qb][kb][i] = key <= pos[qb] ? acc[qb][i] * c2 : -INFINITY;
        }
      }
    }
    bool rescale = false;
    float alpha[kQB];
    bf16x8 pf[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float mx = rows4_max(fmaxf(fmaxf(fmaxf(s[qb][0][0], s[qb][0][1]), fmaxf(s[qb][0][2], s[qb][0][3])),
                                       fmaxf(fmaxf(s[qb][1][0], s[qb][1][1]), fmaxf(s[qb][1][2], s[qb][1][3]))));
      // The reference m_run moves only when some query of the wave gains more
      // than kRefSlack over it (always in the first tile, where m_run = -inf;
      // mx is finite since key 0 <= pos).  Weights 2^(s - m_run) then stay
      // below 2^kRefSlack, which bf16 weights and float32 sums carry without
      // loss, and the accumulators are rescaled only on those tiles.
      alpha[qb] = 1.f;
      if (__any(mx > m_run[qb] + kRefSlack)) {  // the same for the whole wave
        const float m_new = fmaxf(m_run[qb], mx);
        alpha[qb] = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        rescale = true;
      }
      float p[2][4], psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = __builtin_amdgcn_exp2f(s[qb][kb][i] - m_run[qb]);
          psum += p[kb][i];
        }
      l_run[qb] = l_run[qb] * alpha[qb] + rows4_sum(psum);
      // P^T as the B operand: reduction index 8g + jj = key 4g + jj (jj < 4) or 16 + 4g + jj - 4
      const uint32_t pk[4] = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                              pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
      pf[qb] = __builtin_bit_cast(bf16x8, pk);
    }
    if (rescale) {  // one branch per tile; alpha is 1 for a block whose reference stayed
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int db = 0; db < kDh / 16; ++db) {
          o[qb][db][0] *= alpha[qb];
          o[qb][db][1] *= alpha[qb];
          o[qb][db][2] *= alpha[qb];
          o[qb][db][3] *= alpha[qb];
        }
    }
#pragma unroll
    for (int db = 0; db < kDh / 16; ++db) {
      // V^T as the A operand: dimension 16db + q, keys 4g .. 4g+3 and 16 + 4g ..
      // 16 + 4g+3, two transposed reads: lane q of group g addresses key
      // 4g + q/4 (or 16 + 4g + q/4), dimensions 16db + 4(q%4) .. +3
      const uint32_t voff = (4 * g + (q >> 2)) * kVRowB + 2 * (16 * db + 4 * (q & 3));
      const uint64_t vv[2] = {lds_tr4(v_lds, voff), lds_tr4(v_lds, voff + 16 * kVRowB)};
      const bf16x8 vf = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
        o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb], o[qb][db], 0, 0, 0);
    }
  }

  // lane holds O^T[16db + 4g + i][query of block qb]
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    if (!tvalid[qb]) continue;
    const float inv = 1.f / l_run[qb];
    const int64_t row = (static_cast<int64_t>(b) * q_len + t0 + 16 * qb + q) * H + h;
    float* orow = out + row * kDh + 4 * g;
#pragma unroll
    for (int db = 0; db < kDh / 16; ++db) {
      float4_t v = o[qb][db];
      v[0] *= inv;
      v[1] *= inv;
      v[2] *= inv;
      v[3] *= inv;
      *reinterpret_cast<float4_t*>(orow + 16 * db) = v;
    }
    if (lse && g == 0) lse[row] = (m_run[qb] + log2f(l_run[qb])) * kLn2F;
  }
}

}  // namespace

bool is_prefill_shape(const mla_dims& d) {
  return d.dtype == MLA_BF16 && d.d_latent == kDc && d.d_rope == kDr && d.d_head == kDh &&
         d.page_size == kPage;
}

int64_t prefill_workspace_bytes(const mla_dims& d, int batch, int max_pages) {
  return 2 * static_cast<int64_t>(batch) * d.n_heads * max_pages * kPage * kDh * 2;
}

hipError_t prefill_naive(const mla_dims& d, int batch, int q_len, const void* q_nope, const void* q_pe,
                         const void* w_uk, const void* w_uv, const void* kv_cache,
                         const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                         void* workspace, float* out, float* lse, hipStream_t stream) {
  const int max_rows = max_pages * kPage;
  uint16_t* kc = static_cast<uint16_t*>(workspace);
  uint16_t* vc = kc + static_cast<int64_t>(batch) * d.n_heads * max_rows * kDh;
  hipLaunchKernelGGL(materialise_kv_kernel, dim3(d.n_heads, 2, batch), dim3(512), 0, stream,
                     d.n_heads, max_rows, static_cast<const uint16_t*>(kv_cache),
                     block_table, max_pages, seq_lens, static_cast<const uint16_t*>(w_uk),
                     static_cast<const uint16_t*>(w_uv), kc, vc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PrefillTheta theta;
  for (int k = 0; k < kDr / 2; ++k) theta.t[k] = pow(d.rope_base, -2.0 * k / kDr);
  const int wg_tokens = kAttnWaves * kQWave;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3((q_len + wg_tokens - 1) / wg_tokens, d.n_heads, batch),
                     dim3(64 * kAttnWaves), 0,
                     stream, d.n_heads, q_len, max_rows, d.softmax_scale, theta,
                     static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_pe),
                     static_cast<const uint16_t*>(kv_cache), block_table, max_pages, seq_lens, kc, vc, out,
                     lse);
  return hipGetLastError();
}

}  // namespace mla
