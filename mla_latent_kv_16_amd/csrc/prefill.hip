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
//    the caller's workspace.  One workgroup of eight waves per (head,
//    sequence) holds W^UK_i and W^UV_i in registers (32 rows per wave) and
//    streams the sequence's latent rows through an LDS ring by DMA:
//    D^T[32 x 32 rows] = W[32 x 512] . c^T[512 x 32 rows] per wave and tile
//    with v_mfma_f32_32x32x16_bf16, float32 accumulation rounded to bf16 and
//    staged in LDS so that whole rows are stored.
//  * attention: one workgroup of eight waves per (256 query tokens, head,
//    sequence), numbered so that all query blocks of one (sequence, head)
//    run on one XCD at about the same time (they stream the same keys and
//    values, which that XCD's L2 then serves); one wave per 32 queries (two
//    blocks of 16, so that every K or V fragment read from LDS feeds two
//    MFMAs); keys in tiles of 32 staged in LDS for all eight waves (two
//    buffers, K row-major, V transposed), with an online
//    softmax in base 2 whose reference moves only when the running maximum
//    gains more than 2^8 (the accumulators are rescaled only then); the
//    causal mask is applied only on tiles that reach the wave's first query,
//    the scale is folded into the exponent, and the row sums come from the
//    MFMA (an all-ones block times P^T).
//    S^T[16 keys x 16 queries] on MFMA (K rows as A, the query tile as B, 6
//    steps over the 192 dimensions), then O^T[128 x 16 queries] += V^T . P^T
//    with the reduction index running over the keys each lane's score
//    accumulators hold, so P^T needs no reshuffle.
#include <math.h>

#include <algorithm>

#include "decode_common.h"
#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

static_assert(sizeof(RopeTheta::t) / sizeof(double) == kDr / 2, "one angle per RoPE pair");

constexpr float kRefSlack = 8.f;   // log2 units the softmax reference may trail the running maximum
constexpr int kQB = 2;             // 16-query blocks per attention wave
constexpr int kQWave = 16 * kQB;   // query tokens per attention wave
constexpr int kKeyTile = 32;   // keys per attention iteration
constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;

// Maximum over the four lanes q, q+16, q+32, q+48 of a wave.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Row j of sequence b in the paged cache (the caller guarantees j < L_b).
__device__ __forceinline__ const uint16_t* cache_row(const uint16_t* cache, const int32_t* bt, int j) {
  return cache + (static_cast<int64_t>(bt[j >> 6]) * kPage + (j & (kPage - 1))) * kDq;
}

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float float16_t;

// Materialisation, one workgroup per (head h, sequence b): K^C_h = c^KV W^UK_h^T
// and V^C_h = c^KV W^UV_h^T from one pass over the sequence's latent rows.
// Every workgroup of a sequence reads all its latent rows, so the L2-to-CU
// traffic is (latent bytes) x H x (workgroups per head); producing K and V
// together halves it against one workgroup per matrix.  Wave w keeps 32 rows
// of one matrix (rows 32 (w % 4) .. +31 of W^UK_h for w < 4, of W^UV_h
// otherwise) in registers as the A operand of v_mfma_f32_32x32x16_bf16 (32
// k-steps x 8 values = 128 VGPRs); the latent rows stream through a ring of
// kMatSlots LDS tiles of 32 rows, filled by DMA and read as the B operand.
// The products of a tile go through LDS as well, so that each store writes
// four whole 256-byte rows: written straight from the MFMA layout, every store
// would scatter 16-byte pieces over 32 rows, and those partial-line writes
// cost more than the whole latent stream.
constexpr int kMatTile = 32;                       // latent rows per LDS tile
constexpr int kMatSlots = 4;                       // tiles in the ring
constexpr int kMatDma = kMatTile / 8;              // DMA rows per wave per tile
constexpr int kMatStores = 2;                      // global stores per wave per tile
constexpr int kMatRowB = kDc * 2;                  // 1024: latent bytes of a row
constexpr int kMatOutB = 2 * kMatTile * kDh * 2;   // 16 KiB: K and V rows of a tile

// s_waitcnt vmcnt(n') for the largest even n' <= n (n <= 2 kMax)
template <int kMax>
__device__ __forceinline__ void wait_vmcnt_even(int n) {
  if constexpr (kMax == 0) {
    __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
  } else {
    if (n >= 2 * kMax)
      __builtin_amdgcn_s_waitcnt(MLA_VMCNT(2 * kMax));
    else
      wait_vmcnt_even<kMax - 1>(n);
  }
}

__global__ __launch_bounds__(512, 1) void materialise_kv_kernel(
    int H, int max_rows, const uint16_t* __restrict__ cache, const int32_t* __restrict__ block_table,
    int max_pages, const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ w_uk,
    const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc) {
  // ring: tile row r's 16-byte chunk c sits at position c ^ (r % 16), so that
  // a ds_read_b128 cycle (16 lanes of a half-wave: rows n with equal parity of
  // bits 2..4, one chunk) covers all 16 bank groups.  out: two buffers of
  // [matrix][tile row][128 values], chunk c of row r at position c ^ (r % 16).
  __shared__ __attribute__((aligned(1024))) char ring[kMatSlots * kMatTile * kMatRowB];
  __shared__ __attribute__((aligned(1024))) char out[2 * kMatOutB];
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = seq_lens[b];
  if (L <= 0) return;  // uniform over the workgroup, before any barrier
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int n = lane & 31, g2 = lane >> 5;
  const int mat = w >> 2, mb = w & 3;
  // A operand: W row 32 mb + n, latent values 16ks + 8 g2 .. +8
  const uint16_t* wsrc = (mat ? w_uv : w_uk) + (static_cast<int64_t>(h) * kDh + 32 * mb + n) * kDc + 8 * g2;
  bf16x8 a[kDc / 16];
#pragma unroll
  for (int ks = 0; ks < kDc / 16; ++ks) a[ks] = *reinterpret_cast<const bf16x8*>(wsrc + 16 * ks);

  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_pages;
  // split z of gridDim.z takes the tiles z0 .. z0 + ntiles - 1 of the sequence
  // (more workgroups when heads x batch alone would leave CUs idle)
  const int all_tiles = (L + kMatTile - 1) / kMatTile;
  const int per_split = (all_tiles + gridDim.z - 1) / gridDim.z;
  const int z0 = blockIdx.z * per_split;
  const int ntiles = min(per_split, all_tiles - z0);
  if (ntiles <= 0) return;  // uniform over the workgroup, before any barrier
  // the 16 workgroups of a sequence on one XCD (heads h, h + 8, ...) start 16
  // consecutive tiles apart and wrap around, rather than all on one tile
  const int t0 = (h >> 3) % ntiles;
  auto phys = [&](int t) { return z0 + (t + t0 < ntiles ? t + t0 : t + t0 - ntiles); };
  const uint32_t ring_lds = dec::lds_addr_of(ring);
  // wave w copies rows kMatDma w .. +kMatDma of the tile issued t-th, one 1 KiB
  // row per instruction (lane p fetches chunk p ^ (r % 16)); a tile lies inside
  // one 64-row page, and rows past the end repeat row L - 1
  auto issue = [&](int t, int page) {
    const int tp = phys(t);
    const char* pbase = reinterpret_cast<const char*>(cache) + static_cast<int64_t>(page) * kPage * (kDq * 2);
#pragma unroll
    for (int i = 0; i < kMatDma; ++i) {
      const int r = kMatDma * w + i;
      const int j = min(tp * kMatTile + r, L - 1);
      dec::dma16(pbase + (j & (kPage - 1)) * (kDq * 2), 16u * (lane ^ (r & 15)),
                 ring_lds + ((t % kMatSlots) * kMatTile + r) * kMatRowB);
    }
  };
  // Vector-memory operations of this wave issued after tile t's DMA, before
  // the wait for it (they complete in issue order): the DMA of tiles t+1 ..
  // t+kMatSlots-2, and the stores that iterations t-kMatSlots+1 .. t-1 made
  // of the tile before each of them.
  auto wait_tile = [&](int t) {
    const int dma_after = min(t + kMatSlots - 2, ntiles - 1) - t;
    const int store_iters = t == 0 ? 0 : t - max(t - kMatSlots + 1, 1);
    wait_vmcnt_even<(kMatDma * (kMatSlots - 2) + kMatStores * (kMatSlots - 1)) / 2>(
        kMatDma * dma_after + kMatStores * store_iters);
  };
  static_assert(kMatDma % 2 == 0 && kMatStores % 2 == 0, "even wait counts");

  // stores of tile t from out buffer t % 2: wave w writes rows 8 mb + 4s ..
  // +3 (s < 2) of matrix `mat`, 16 bytes per lane, 1 KiB per instruction; the
  // whole tile is written (rows from L on hold row L - 1's products and lie
  // inside the workspace, which has max_pages * 64 rows)
  uint16_t* dst = (mat ? vc : kc) + (static_cast<int64_t>(b) * H + h) * max_rows * kDh;
  auto store_tile = [&](int t) {
    const char* ob = out + (t & 1) * kMatOutB + mat * (kMatTile * kDh * 2);
    const int c = lane & 15;
#pragma unroll
    for (int s2 = 0; s2 < kMatStores; ++s2) {
      const int r = 8 * mb + 4 * s2 + (lane >> 4);
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(ob + r * (kDh * 2) + 16 * (c ^ (r & 15)));
      *reinterpret_cast<bf16x8*>(dst + static_cast<int64_t>(phys(t) * kMatTile + r) * kDh + 8 * c) = v;
    }
  };

  for (int t = 0; t < kMatSlots - 1 && t < ntiles; ++t) issue(t, bt[phys(t) >> 1]);
  int next_page = kMatSlots - 1 < ntiles ? bt[phys(kMatSlots - 1) >> 1] : 0;
  // B operand: tile row n, chunk 2ks + g2, at position 2ks ^ (g2 ^ (n % 16))
  const int y = g2 ^ (n & 15);
  for (int t = 0; t < ntiles; ++t) {
    wait_tile(t);
    // tile t is in LDS; tile t-1's ring slot is free; tile t-1's products are
    // in out buffer (t-1) % 2, and buffer t % 2 has been stored
    __syncthreads();
    if (t + kMatSlots - 1 < ntiles) {
      issue(t + kMatSlots - 1, next_page);
      if (t + kMatSlots < ntiles) next_page = bt[phys(t + kMatSlots) >> 1];
    }
    const char* rb = ring + ((t % kMatSlots) * kMatTile + n) * kMatRowB;
    float16_t acc = {};
#pragma unroll
    for (int ks = 0; ks < kDc / 16; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          a[ks], *reinterpret_cast<const bf16x8*>(rb + 16 * ((2 * ks) ^ y)), acc, 0, 0, 0);
    if (t > 0) store_tile(t - 1);
    // lane holds values 32 mb + 8i + 4 g2 .. +3 (i < 4) of tile row n: 8 bytes
    // of chunk 4 mb + i
    char* orow = out + (t & 1) * kMatOutB + mat * (kMatTile * kDh * 2) + n * (kDh * 2) + 8 * g2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = pack_bf16x2(acc[4 * i], acc[4 * i + 1]), hi = pack_bf16x2(acc[4 * i + 2], acc[4 * i + 3]);
      *reinterpret_cast<uint64_t*>(orow + 16 * ((4 * mb + i) ^ (n & 15))) = (static_cast<uint64_t>(hi) << 32) | lo;
    }
  }
  __syncthreads();
  store_tile(ntiles - 1);
}

// K tile: 32 keys x 192 dimensions, rows padded to 400 bytes.  V tile: 32 keys
// x 128 dimensions, rows padded to 288 bytes, read transposed with
// ds_read_b64_tr_b16 (a 16-lane group reads 4 keys x 16 dimensions and each
// lane receives the 4 keys of one dimension; the 32-byte row shift puts the 8
// rows a half-wave reads in distinct bank groups).
constexpr int kKRowB = 2 * (kDh + kDr) + 16;  // 400
constexpr int kVRowB = 2 * kDh + 32;          // 288
constexpr int kAttnWaves = 8;                  // query tiles per workgroup

__device__ __forceinline__ uint64_t lds_tr4(const char* lds, uint32_t off) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)((__attribute__((address_space(3))) const char*)lds + off));
  return __builtin_bit_cast(uint64_t, v);
}

__global__ __launch_bounds__(64 * kAttnWaves, 1) void prefill_attn_kernel(
    int H, int batch, int q_len, int max_rows, float scale, RopeTheta theta,
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const uint16_t* __restrict__ cache, const int32_t* __restrict__ block_table, int max_pages,
    const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, float* __restrict__ out, float* __restrict__ lse) {
  // two buffers: the next tile is stored while the waves compute on this one
  __shared__ __attribute__((aligned(16))) char ks_buf[2][kKeyTile * kKRowB];
  __shared__ __attribute__((aligned(16))) char v_buf[2][kKeyTile * kVRowB];
  // block -> (query block, sequence and head): the query blocks of one
  // (sequence, head) share an XCD (blocks i and i + 8 do) and follow each
  // other in dispatch order
  const int n_qblk = (q_len + kAttnWaves * kQWave - 1) / (kAttnWaves * kQWave);
  int bh, qblk;
  dec::block_to_item(blockIdx.x, batch * H, n_qblk, bh, qblk);
  const int b = bh / H, h = bh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, q = lane & 15;
  const int L = seq_lens[b];
  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_pages;
  const int t0 = (qblk * kAttnWaves + w) * kQWave;   // this wave's first query
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
  const int tw_end = min((qblk + 1) * kAttnWaves * kQWave, q_len);
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
  // position of the wave's first query: a tile whose last key is at most this
  // needs no causal mask (a tile holding keys at or past L never qualifies)
  const int p_first = L - q_len + min(t0, q_len - 1);
  // all-ones A operand: O^T's extra block 1 . P^T gives every query's row sum
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = static_cast<__bf16>(1.0f);
  const uint16_t* kh = kc + (static_cast<int64_t>(b) * H + h) * max_rows * kDh;
  const uint16_t* vh = vc + (static_cast<int64_t>(b) * H + h) * max_rows * kDh;
  float4_t o[kQB][kDh / 16];
  float m_run[kQB];
  float4_t lacc[kQB];  // row sums (every element of a lane: its query's)
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
    for (int db = 0; db < kDh / 16; ++db) o[qb][db] = float4_t{0.f, 0.f, 0.f, 0.f};
    m_run[qb] = -INFINITY;
    lacc[qb] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Tile staging, software-pipelined over two LDS buffers: the 512 threads
  // hold the next tile in registers (K^C and V: key i/16, chunk i%16; k^R,
  // threads < 256: key i/8, chunk i%8), store it into the free buffer at the
  // top of an iteration and load the one after it, then the waves compute on
  // the buffer stored there.  One barrier per tile: a buffer is stored again
  // two iterations after it was read, with a barrier in between.
  static_assert(kKeyTile * 16 == 64 * kAttnWaves && kKeyTile * 8 == 32 * kAttnWaves, "staging split");
  bf16x8 rk, rv, rr;
  const bool rope_thread = threadIdx.x < kKeyTile * 8;
  auto load_tile = [&](int k0) {
    const int i = threadIdx.x;
    const int key = min(k0 + (i >> 4), L - 1);
    rk = *reinterpret_cast<const bf16x8*>(kh + static_cast<int64_t>(key) * kDh + 8 * (i & 15));
    rv = *reinterpret_cast<const bf16x8*>(vh + static_cast<int64_t>(key) * kDh + 8 * (i & 15));
    if (rope_thread) {
      const int kr = min(k0 + (i >> 3), L - 1);
      rr = *reinterpret_cast<const bf16x8*>(cache_row(cache, bt, kr) + kDc + 8 * (i & 7));
    }
  };
  auto store_tile = [&](int buf) {
    const int i = threadIdx.x;
    *reinterpret_cast<bf16x8*>(ks_buf[buf] + (i >> 4) * kKRowB + 16 * (i & 15)) = rk;
    *reinterpret_cast<bf16x8*>(v_buf[buf] + (i >> 4) * kVRowB + 16 * (i & 15)) = rv;
    if (rope_thread)
      *reinterpret_cast<bf16x8*>(ks_buf[buf] + (i >> 3) * kKRowB + 2 * kDh + 16 * (i & 7)) = rr;
  };
  load_tile(0);
  for (int k0 = 0, it = 0; k0 <= p_wg; k0 += kKeyTile, ++it) {
    store_tile(it & 1);
    if (k0 + kKeyTile <= p_wg) load_tile(k0 + kKeyTile);
    __syncthreads();
    if (k0 > p_wave) continue;  // every key of the tile lies after this wave's queries
    const char* ks_lds = ks_buf[it & 1];
    const char* v_lds = v_buf[it & 1];

    // S^T for keys k0 + 16kb + row, queries of block qb: lane holds keys
    // 16kb + 4g + i.  Each row fragment read from LDS feeds one MFMA per
    // query block.
    const bool diag = k0 + kKeyTile - 1 > p_first;  // the same for the whole wave
    // raw scores q . K (not yet scaled); -inf where masked
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
          s[qb][kb][i] = (!diag || key <= pos[qb]) ? acc[qb][i] : -INFINITY;
        }
      }
    }
    bool rescale = false;
    float alpha[kQB];
    bf16x8 pf[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float mx = c2 * rows4_max(fmaxf(fmaxf(fmaxf(s[qb][0][0], s[qb][0][1]), fmaxf(s[qb][0][2], s[qb][0][3])),
                                            fmaxf(fmaxf(s[qb][1][0], s[qb][1][1]), fmaxf(s[qb][1][2], s[qb][1][3]))));
      // The reference m_run (log2 units) moves only when some query of the
      // wave gains more than kRefSlack over it (always in the first tile,
      // where m_run = -inf; mx is finite since key 0 <= pos).  Weights
      // 2^(s - m_run) then stay below 2^kRefSlack, which bf16 weights and
      // float32 sums carry without loss, and the accumulators are rescaled
      // only on those tiles.
      alpha[qb] = 1.f;
      if (__any(mx > m_run[qb] + kRefSlack)) {  // the same for the whole wave
        const float m_new = fmaxf(m_run[qb], mx);
        alpha[qb] = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        rescale = true;
      }
      float p[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][i], c2, -m_run[qb]));
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
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        lacc[qb][0] *= alpha[qb];
        lacc[qb][1] *= alpha[qb];
        lacc[qb][2] *= alpha[qb];
        lacc[qb][3] *= alpha[qb];
      }
    }
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
      lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[qb], lacc[qb], 0, 0, 0);
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
    const float l_sum = lacc[qb][0];
    const float inv = 1.f / l_sum;
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
    if (lse && g == 0) lse[row] = (m_run[qb] + log2f(l_sum)) * kLn2F;
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
  // one workgroup per (head, sequence), each sequence's rows split further
  // when that leaves CUs idle, keeping at least 8 tiles per split
  const int64_t pairs = static_cast<int64_t>(d.n_heads) * batch;
  const int max_tiles = max_pages * (kPage / kMatTile);
  const int splits = static_cast<int>(
      std::max<int64_t>(1, std::min<int64_t>((256 + pairs - 1) / pairs, max_tiles / 8)));
  hipLaunchKernelGGL(materialise_kv_kernel, dim3(d.n_heads, batch, splits), dim3(512), 0, stream,
                     d.n_heads, max_rows, static_cast<const uint16_t*>(kv_cache),
                     block_table, max_pages, seq_lens, static_cast<const uint16_t*>(w_uk),
                     static_cast<const uint16_t*>(w_uv), kc, vc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RopeTheta theta;
  for (int k = 0; k < kDr / 2; ++k) theta.t[k] = pow(d.rope_base, -2.0 * k / kDr);
  const int wg_tokens = kAttnWaves * kQWave;
  const int64_t blocks = static_cast<int64_t>((q_len + wg_tokens - 1) / wg_tokens) * d.n_heads * batch;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(64 * kAttnWaves), 0,
                     stream, d.n_heads, batch, q_len, max_rows, d.softmax_scale, theta,
                     static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_pe),
                     static_cast<const uint16_t*>(kv_cache), block_table, max_pages, seq_lens, kc, vc, out,
                     lse);
  return hipGetLastError();
}

}  // namespace mla
