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

#include "decode_common.h"
#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

static_assert(sizeof(RopeTheta::t) / sizeof(double) == kDr / 2, "one angle per RoPE pair");

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
    int batch, int H, RopeTheta theta_k, const uint16_t* __restrict__ q_nope,
    const uint16_t* __restrict__ q_pe, const int32_t* __restrict__ positions,
    const char* __restrict__ w_uk, uint16_t* __restrict__ q_abs) {
  constexpr int kCols = 128, kTileRow = kCols * 2;  // 256 bytes
  constexpr int kStageRow = kTileRow + 16;          // output staging row, padded
  __shared__ __attribute__((aligned(1024))) char lds[kDh * kTileRow];
  __shared__ __attribute__((aligned(16))) char stage[4 * 16 * kStageRow];
  const uint32_t lds_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));
  int h, quarter;
  xcd_split(blockIdx.x, 4, h, quarter);
  const int c0 = quarter * kCols;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, q = lane & 15;

  const int b0 = blockIdx.y * 64;
  const int nb = min(64, batch - b0);
  // B operand: q^C of sequence b = b0 + 16w + q, values 32ks + 8g .. +8 (a
  // clamped index past the batch; those columns are not stored)
  const int b = min(b0 + 16 * w + q, batch - 1);
  const uint16_t* qrow = q_nope + (static_cast<int64_t>(b) * H + h) * kDh + 8 * g;
  bf16x8 qn[4];
  if (w < 2) {
    // Waves 0 and 1 stage W^UK_h[:, c0:c0+128], rows 64w .. 64w+63: LDS chunk
    // p = row * 16 + pc holds chunk pc ^ tsw(row).
    const char* wh = w_uk + static_cast<int64_t>(h) * kDh * (kDc * 2) + c0 * 2;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p = (16 * w + i) * 64 + lane;
      const int row = p >> 4, pc = p & 15;
      dec::dma16(wh, row * (kDc * 2) + 16 * (pc ^ tsw(row)), lds_base + (16 * w + i) * 1024);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qn[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  } else {
    // Waves 2 and 3: the RoPE part, float64 angle, float32 rotation, while the
    // tile is in flight (the load counter is per wave, so waiting for these
    // loads does not wait for the tile).  The four quarter-workgroups of a head
    // share the (sequence, pair) list: thread t keeps pair k = t % 32 of four
    // sequences.  Loads are unconditional, from a clamped sequence index, so
    // that no branch forces a wait between them.
    // (q^C first: the rotation's wait then covers it too, and no load of
    // these waves is left pending where the two roles' code joins)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qn[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
    const int t = threadIdx.x - 128;
    const int k = t & (kDr / 2 - 1);
    const int bi0 = quarter * 8 + (t >> 5);
    constexpr int kPer = 4;
    int pos[kPer];
    uint32_t xy[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int bi = min(bi0 + 4 * (j & 1) + 32 * (j >> 1), nb - 1);
      const int64_t r = static_cast<int64_t>(b0 + bi) * H + h;
      pos[j] = positions[b0 + bi];
      xy[j] = *reinterpret_cast<const uint32_t*>(q_pe + r * kDr + 2 * k);
    }
    const double theta = theta_k.t[k];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int bi = bi0 + 4 * (j & 1) + 32 * (j >> 1);
      float sn, c;
      sincos_reduced(static_cast<double>(pos[j]) * theta, sn, c);
      const int64_t r = static_cast<int64_t>(b0 + bi) * H + h;
      const float x0 = bf16_bits_to_f32(static_cast<uint16_t>(xy[j] & 0xffffu));
      const float x1 = bf16_bits_to_f32(static_cast<uint16_t>(xy[j] >> 16));
      const uint32_t y = pack_bf16x2(x0 * c - x1 * sn, x0 * sn + x1 * c);
      if (bi < nb) *reinterpret_cast<uint32_t*>(q_abs + r * kDq + kDc + 2 * k) = y;
    }
  }

  __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
  __syncthreads();
  if (16 * w >= nb) return;  // no sequence for this wave (no barrier follows)

  // A operand rows d = 32ks + 8g + s (+4), columns 16cb + 4(q%4) of the tile:
  // source-lane role q -> row 8g + q/4 of the k block, chunk 2cb + (q%4)/2.
  const int arow = 8 * g + (q >> 2);
  const int sw0 = tsw(arow), sw1 = tsw(arow + 4);
  float4_t accs[kCols / 16];
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
    accs[cb] = acc;  // q~[c0 + 16cb + 4g + i] of sequence b
  }
  // Through a wave-private LDS block (16 sequences x 128 columns, rows padded to
  // 272 bytes) so that the stores write whole 256-byte row segments, 16 bytes
  // per lane.  LDS accesses of one wave complete in order: no barrier.
  char* st = stage + w * (16 * kStageRow);
#pragma unroll
  for (int cb = 0; cb < kCols / 16; ++cb) {
    const uint32_t lo = pack_bf16x2(accs[cb][0], accs[cb][1]);
    const uint32_t hi = pack_bf16x2(accs[cb][2], accs[cb][3]);
    *reinterpret_cast<uint64_t*>(st + q * kStageRow + 32 * cb + 8 * g) = (static_cast<uint64_t>(hi) << 32) | lo;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = (lane >> 4) + 4 * j, c = lane & 15;
    const float4_t v = *reinterpret_cast<const float4_t*>(st + rr * kStageRow + 16 * c);
    const int bb = b0 + 16 * w + rr;
    if (bb < batch)
      *reinterpret_cast<float4_t*>(q_abs + (static_cast<int64_t>(bb) * H + h) * kDq + c0 + 8 * c) = v;
  }
}

// ---------------------------------------------------------------------------
// out_proj: o^T[128 x r] = W^UV_h[128 x 512] . o~^T[512 x r], one workgroup of
// eight waves per (head, kOutRows = 32, 16, 8 or 4 query rows).  Blocks (h, group)
// and (h, group') run on one XCD (grid x = heads, a multiple of 8), so W^UV_h
// comes from HBM once and from that XCD's L2 for the other groups.  The
// float32 o~ of the rows is staged once in LDS as bf16 hi + lo (lo = bf16(x - hi)), rows of
// 1 KiB with 16-byte chunk c at position c ^ 2 (r % 8): the B-operand reads
// (16 rows x one chunk per quarter-wave) then hit distinct bank groups.  Wave
// w owns output rows 16w .. 16w+15 for all the rows (an accumulator per 16), its
// W^UV rows read straight from global memory.
//
// With kMerge the workgroup first merges the split-KV partials of its rows
// (the log-sum-exp combine, same arithmetic and order as combine_512_kernel,
// so o~ is bit-identical) and stages the merged o~ instead of reading it; it
// also writes o~ and lse when those pointers are set.  Rows are query rows
// r = b * q_len + t; item s holds row r's partial at s * q_len + t.
// ---------------------------------------------------------------------------
constexpr int kOutThreads = 512;

template <bool kMerge, int kOutRows = 32>
__global__ __launch_bounds__(kOutThreads) void out_proj_kernel(int rows, int H, int q_len,
                                                               const int32_t* __restrict__ offs,
                                                               const float* __restrict__ o_part,
                                                               const float* __restrict__ lse_part,
                                                               float* __restrict__ o_lat,
                                                               float* __restrict__ lse_out,
                                                               const uint16_t* __restrict__ w_uv,
                                                               float* __restrict__ out) {
  constexpr int kRowBlocks = kOutRows >= 16 ? kOutRows / 16 : 1;
  // one bf16 copy of the staged o~; at 8 rows the MFMA's 16-row block also
  // reads rows 8..15, whose outputs are dropped
  constexpr int kOutHalfBytes = 16 * kRowBlocks * kDc * 2;
  constexpr int kOutF4 = kOutRows * (kDc / 4) / kOutThreads;  // float4 per thread: 8, 4, 2 or 1
  static_assert(kOutF4 >= 1, "a thread stages whole float4s of at least one row");
  __shared__ __attribute__((aligned(16))) char lds[2 * kOutHalfBytes];  // [hi | lo][r][512]
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, q = lane & 15;
  const int r0 = blockIdx.y * kOutRows;
  const int nr = min(kOutRows, rows - r0);

  // A operand: W^UV row 16w + q, values 32ks + 8g .. +8
  const uint16_t* wrow = w_uv + (static_cast<int64_t>(h) * kDh + 16 * w + q) * kDc + 8 * g;
  bf16x8 a[16];
  auto load_w = [&]() {
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) a[ks] = *reinterpret_cast<const bf16x8*>(wrow + 32 * ks);
  };

  // thread t stages float4 column 4 (t % 128) of rows t / 128 + 4 i, i < kOutF4
  const int c4 = 4 * (threadIdx.x & 127);
  const int rl0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 7);  // the same for a whole wave
  float4_t v[kOutF4];
  if constexpr (kMerge) {
    // Row rl = rl0 + 4i has items s0[i] .. s0[i] + ns[i] - 1 (the same for
    // every lane of a wave).  The loads go out in three rounds, each in
    // flight as a whole: (1) the split offsets of the workgroup's sequences,
    // one per lane (per-row scalar loads were issued one round trip apart),
    // then W^UV; (2) the lse of up to kChunk items of every row, one per
    // lane, and the partials of the first kPair items of every row (16 float4
    // per thread); (3) the partials of later items, kPair at a time.  M is a
    // max over the lanes of a row; the weights exp(lse - M), Z and the
    // weighted sum are taken in item order, each row's arithmetic exactly the
    // combine's, so o~ matches mla_combine bit for bit.
    // Loads are unconditional (a row past the end, or an item past a row's
    // last, reads the row's last item and the value is then replaced), so no
    // branch separates them; the planner gives every sequence at least one
    // item.
    constexpr int kPair = 16 / kOutF4;   // items per load round of partials: 2, 4, 8 or 16
    constexpr int kChunk = 64 / kOutF4;  // items per lse load: 8, 16, 32 or 64
    // (a row's sequence: one query token per sequence is the common case, and
    // it needs no division)
    const bool one = q_len == 1;
    const int b_first = one ? r0 : r0 / q_len;
    const int nseq = (one ? r0 + nr - 1 : (r0 + nr - 1) / q_len) - b_first + 1;  // <= kOutRows < 64
    const int off_v = offs[b_first + min(lane, nseq)];     // offs[b_first + lane]
    load_w();
    int s0[kOutF4], ns[kOutF4], nv[kOutF4], tq[kOutF4];
    int nsmax = 0;
#pragma unroll
    for (int i = 0; i < kOutF4; ++i) {
      const int rl = rl0 + 4 * i;
      const int r = r0 + min(rl, nr - 1);
      const int b = one ? r : r / q_len;
      tq[i] = r - b * q_len;
      s0[i] = __builtin_amdgcn_readlane(off_v, b - b_first);
      nv[i] = __builtin_amdgcn_readlane(off_v, b - b_first + 1) - s0[i];
      ns[i] = rl < nr ? nv[i] : 0;
      nsmax = max(nsmax, ns[i]);
    }
    // lane l holds the lse of item kc + l / kOutF4 of row l % kOutF4
    const int li = lane % kOutF4, lk = lane / kOutF4;
    int s0_l = s0[0], nv_l = nv[0], ns_l = ns[0], tq_l = tq[0];
#pragma unroll
    for (int i = 1; i < kOutF4; ++i) {
      const bool mine = li == i;
      s0_l = mine ? s0[i] : s0_l;
      nv_l = mine ? nv[i] : nv_l;
      ns_l = mine ? ns[i] : ns_l;
      tq_l = mine ? tq[i] : tq_l;
    }
    auto lse_raw = [&](int kc) -> float {  // the load; lse_sel masks it
      const int kk = max(0, min(kc + lk, nv_l - 1));
      return lse_part[(static_cast<int64_t>(s0_l + kk) * q_len + tq_l) * H + h];
    };
    auto lse_sel = [&](int kc, float l) { return kc + lk < ns_l ? l : -INFINITY; };
    auto lse_at = [&](int kc) { return lse_sel(kc, lse_raw(kc)); };
    auto row_max = [&](float x) {
#pragma unroll
      for (int m = kOutF4; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
      return x;
    };
    auto prow = [&](int i, int k) -> int64_t {  // row of item min(k, last) of row i
      const int kk = max(0, min(k, nv[i] - 1));
      return (static_cast<int64_t>(s0[i] + kk) * q_len + tq[i]) * H + h;
    };
    float4_t x[kPair][kOutF4];
    auto load_pair = [&](int k) {
#pragma unroll
      for (int u = 0; u < kPair; ++u)
#pragma unroll
        for (int i = 0; i < kOutF4; ++i) {
          const float4_t xv = *reinterpret_cast<const float4_t*>(o_part + prow(i, k + u) * kDc + c4);
          x[u][i] = k + u < ns[i] ? xv : float4_t{0.f, 0.f, 0.f, 0.f};
        }
    };
    float lv = lse_raw(0);
    __builtin_amdgcn_sched_barrier(0);  // the lse load goes out before the partials
    load_pair(0);
    lv = lse_sel(0, lv);
    float mv = row_max(lv);  // M of the lane's row, on every lane of that row
    for (int kc = kChunk; kc < nsmax; kc += kChunk) mv = fmaxf(mv, row_max(lse_at(kc)));
    float wv = expf(lv - mv);  // weight of the lane's (row, item)
    float M[kOutF4], Z[kOutF4];
#pragma unroll
    for (int i = 0; i < kOutF4; ++i) {
      M[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mv), i));
      Z[i] = 0.f;
      v[i] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int k = 0; k < nsmax; k += kPair) {
      if (k > 0) {
        if (k % kChunk == 0) wv = expf(lse_at(k) - mv);
        load_pair(k);
      }
#pragma unroll
      for (int i = 0; i < kOutF4; ++i)
#pragma unroll
        for (int u = 0; u < kPair; ++u) {
          if (k + u >= ns[i]) continue;
          const float wgt = __int_as_float(
              __builtin_amdgcn_readlane(__float_as_int(wv), (k + u) % kChunk * kOutF4 + i));
          Z[i] += wgt;
          v[i][0] = fmaf(wgt, x[u][i][0], v[i][0]);
          v[i][1] = fmaf(wgt, x[u][i][1], v[i][1]);
          v[i][2] = fmaf(wgt, x[u][i][2], v[i][2]);
          v[i][3] = fmaf(wgt, x[u][i][3], v[i][3]);
        }
    }
#pragma unroll
    for (int i = 0; i < kOutF4; ++i) {
      const int rl = rl0 + 4 * i;
      if (rl < nr) {
        const float inv = 1.f / Z[i];
        v[i][0] *= inv;
        v[i][1] *= inv;
        v[i][2] *= inv;
        v[i][3] *= inv;
        const int64_t ro = static_cast<int64_t>(r0 + rl) * H + h;
        if (o_lat) *reinterpret_cast<float4_t*>(o_lat + ro * kDc + c4) = v[i];
        if (lse_out && c4 == 0) lse_out[ro] = M[i] + logf(Z[i]);
      } else {
        v[i] = float4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  } else {
    load_w();
#pragma unroll
    for (int i = 0; i < kOutF4; ++i) {
      const int rl = rl0 + 4 * i;
      v[i] = rl < nr ? *reinterpret_cast<const float4_t*>(o_lat + (static_cast<int64_t>(r0 + rl) * H + h) * kDc + c4)
                     : float4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int i = 0; i < kOutF4; ++i) {
    const int rl = rl0 + 4 * i;
    const uint32_t off = rl * (kDc * 2) + 16 * ((c4 >> 3) ^ (2 * (rl & 7))) + 2 * (c4 & 7);
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
  __syncthreads();

  // B operand: row 16bb + q, values 32ks + 8g .. +8 (chunk 4ks + g)
  float4_t acc[kRowBlocks] = {};
  const uint32_t brow = q * (kDc * 2);
  const int bsw = 2 * (q & 7);
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const uint32_t col = 16 * ((4 * ks + g) ^ bsw);
#pragma unroll
    for (int bb = 0; bb < kRowBlocks; ++bb) {
      const uint32_t off = bb * 16 * (kDc * 2) + brow + col;
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(lds + off);
      const bf16x8 bl = *reinterpret_cast<const bf16x8*>(lds + kOutHalfBytes + off);
      acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], bh, acc[bb], 0, 0, 0);
      acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], bl, acc[bb], 0, 0, 0);
    }
  }
  // lane holds o[r0 + 16bb + q][h][16w + 4g + i]
#pragma unroll
  for (int bb = 0; bb < kRowBlocks; ++bb) {
    const int rl = 16 * bb + q;
    if (rl < nr)
      *reinterpret_cast<float4_t*>(out + (static_cast<int64_t>(r0 + rl) * H + h) * kDh + 16 * w + 4 * g) = acc[bb];
  }
}

}  // namespace

int64_t absorb_fast_groups(int64_t batch) { return (batch + 63) / 64; }

int64_t out_proj_fast_groups(int64_t rows) { return (rows + 31) / 32; }

int combine_out_proj_rows_per_group(int n_heads, int64_t rows) {
  // Query rows per workgroup: the largest of 32, 16, 8 that still gives
  // 256 workgroups (one per CU), else 4.  A workgroup pulls every item's
  // partial of its rows and all of W^UV_h through one CU, so few large
  // workgroups are slow: at 16 heads x 32 rows, 16 workgroups of 32 rows
  // took 26 us.
  for (int cand : {32, 16, 8})
    if (n_heads * ((rows + cand - 1) / cand) >= 256) return cand;
  return 4;
}

hipError_t absorb_fast(const mla_dims& d, int batch, const void* q_nope, const void* q_pe,
                       const int32_t* positions, const void* w_uk, void* q_abs,
                       hipStream_t stream) {
  const int64_t groups = absorb_fast_groups(batch);
  if (groups > 65535 || d.n_heads % 8 != 0) return hipErrorInvalidValue;
  RopeTheta theta;
  for (int k = 0; k < kDr / 2; ++k) theta.t[k] = pow(d.rope_base, -2.0 * k / kDr);
  hipLaunchKernelGGL(absorb_kernel, dim3(d.n_heads * 4, static_cast<uint32_t>(groups)), dim3(256), 0, stream, batch,
                     d.n_heads, theta, static_cast<const uint16_t*>(q_nope),
                     static_cast<const uint16_t*>(q_pe), positions,
                     static_cast<const char*>(w_uk), static_cast<uint16_t*>(q_abs));
  return hipGetLastError();
}

hipError_t out_proj_fast(const mla_dims& d, int batch, const float* o_latent, const void* w_uv,
                         float* out, hipStream_t stream) {
  constexpr int kOutRows = 32;
  const int64_t groups = out_proj_fast_groups(batch);
  if (groups > 65535 || d.n_heads % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((out_proj_kernel<false, kOutRows>), dim3(d.n_heads, static_cast<uint32_t>(groups)), dim3(kOutThreads), 0, stream, batch,
                     d.n_heads, 1, nullptr, nullptr, nullptr, const_cast<float*>(o_latent), nullptr,
                     static_cast<const uint16_t*>(w_uv), out);
  return hipGetLastError();
}

hipError_t combine_out_proj_fast(const mla_dims& d, int batch, int q_len, const int32_t* split_offsets,
                                 const float* o_part, const float* lse_part, const void* w_uv,
                                 float* out, float* o_latent, float* lse, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(batch) * q_len;
  if (d.n_heads % 8 != 0) return hipErrorInvalidValue;
  const int R = combine_out_proj_rows_per_group(d.n_heads, rows);
  const int64_t groups = (rows + R - 1) / R;
  if (groups > 65535) return hipErrorInvalidValue;
  const dim3 grid(d.n_heads, static_cast<uint32_t>(groups));
  const int nrows = static_cast<int>(rows);
  const uint16_t* w = static_cast<const uint16_t*>(w_uv);
  if (R == 32)
    hipLaunchKernelGGL((out_proj_kernel<true, 32>), grid, dim3(kOutThreads), 0, stream, nrows, d.n_heads, q_len,
                       split_offsets, o_part, lse_part, o_latent, lse, w, out);
  else if (R == 16)
    hipLaunchKernelGGL((out_proj_kernel<true, 16>), grid, dim3(kOutThreads), 0, stream, nrows, d.n_heads, q_len,
                       split_offsets, o_part, lse_part, o_latent, lse, w, out);
  else if (R == 8)
    hipLaunchKernelGGL((out_proj_kernel<true, 8>), grid, dim3(kOutThreads), 0, stream, nrows, d.n_heads, q_len,
                       split_offsets, o_part, lse_part, o_latent, lse, w, out);
  else
    hipLaunchKernelGGL((out_proj_kernel<true, 4>), grid, dim3(kOutThreads), 0, stream, nrows, d.n_heads, q_len,
                       split_offsets, o_part, lse_part, o_latent, lse, w, out);
  return hipGetLastError();
}

}  // namespace mla
