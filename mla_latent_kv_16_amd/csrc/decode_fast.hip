// Split-KV MLA decode over the paged latent cache, gfx950 fast path.
//
// Shape: bf16, d_c = 512, d_h^R = 64 (576-value rows), 64-token pages.
// What one work item computes (page "DeepSeek-V2/V3：大模型的两张账", "第一张账"
// and the RoPE section; page "DeepSeek V2 技术解析" 2.2.2): for every head i,
//   s_ij = scale * (q_abs_i . row_j),  row_j = [c^KV_j | k^R_j]
//   o_i  = sum_j softmax_j(s_ij) * c^KV_j      (latent space)
// All heads read the same rows, so per slice of tokens this is two dense
// contractions, S^T = Rows . Q^T  ([tokens x 576] . [576 x heads]) and
// O^T += C^T . P^T ([512 x tokens] . [tokens x heads]), both on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16) with float32 accumulation.
//
// Data movement
//  * Rows stream HBM -> LDS with global_load_lds_dwordx4 (16 bytes per lane,
//    no VGPR round trip) into a ring of 32-token slots (36,864 bytes each),
//    two slices ahead of the one being scored.  A slot is stored as 4 x 9
//    tiles of 8 rows x 128 bytes (1 KiB, one DMA instruction each); inside a
//    tile the 16-byte chunk `ch` of row `t` sits at chunk position
//    ch ^ swz(t) (see swz).  Each lane picks which global chunk it fetches,
//    so the swizzle costs nothing at load time, and one per-lane offset plus
//    a scalar base address every tile of a wave.
//  * The LDS holds only four slots, so the stream is deepened through the L2:
//    the V waves without DMA touch one 4-byte word of every 128-byte line of
//    the slice MLA_PREFETCH_D ahead (the even lines in one workgroup of the
//    pair, the odd ones in the other), with a load whose data lands in a junk
//    LDS line; by the time that slice's DMA is issued its rows are in the L2.
//  * QK^T operands: a lane reads 16 contiguous bytes (8 latent values of one
//    token) with ds_read_b128.
//  * PV operands: C^T needs 8 tokens of one latent column per lane; two
//    ds_read_b64_tr_b16 (4 tokens x 16 columns per 16-lane group, transposed
//    in the LDS crossbar) deliver them.  The MFMA's reduction index k is
//    permuted (k -> token sigma(g, k), see below) so that the QK^T
//    accumulators of a lane already hold the P^T operand of the same lane.
//
// Work split, H = 128: two workgroups per work item, one per half of the
// heads (see decode_h128_kernel), each with sixteen waves in two roles:
//  * eight S waves: scores of 16 heads over one 16-token half of every slice
//    (Q fragments stay in 72 VGPRs), turned into bf16 weights and put in a
//    4 KiB LDS exchange buffer;
//  * eight V waves: the latent PV of 64 columns for the workgroup's 64 heads
//    (64 accumulators), so each transposed C^T fragment feeds 4 MFMAs; four
//    of them also run the DMA, the other four the L2 prefetch.
//  The V waves run one slice behind the S waves; one workgroup barrier per
//  slice.  H = 16 (decode_h16_kernel): one workgroup of four waves per item,
//  each scoring all 16 heads itself.
//
// Softmax in base 2 against a fixed reference per head: the maximum of the
// item's first slice.  Weights 2^(x - m_ref) may exceed 1 by up to 2^20, which
// float32 accumulators and bf16 weights carry without loss of relative
// precision, so the accumulators are never rescaled in registers.  If a
// later slice exceeds the reference by more than that, the workgroup agrees on
// it through an LDS vote after the pass, takes the exact per-head maxima in a
// scores-only pass and redoes the item against them; the result is the same
// softmax either way.
#include <math.h>
#include <stdlib.h>

#include <type_traits>

#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kRowBytes = kDq * 2;             // 1152
constexpr int kSliceTok = 32;
constexpr int kSlotBytes = kSliceTok * kRowBytes;  // 36,864
constexpr int kStages = 4;
constexpr int kDmaWaves = 4;
constexpr int kLoadsPerWave = kSlotBytes / 1024 / kDmaWaves;  // 9 instructions of 1 KiB
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMaxJumpDefault = 20.0f;  // log2 units; see the softmax note above

// Pipelining depths (steps of LDS reads issued ahead of their MFMAs).
#ifndef MLA_QK_AHEAD
#define MLA_QK_AHEAD 4
#endif
#ifndef MLA_PV_AHEAD
#define MLA_PV_AHEAD 2
#endif
#ifndef MLA_S_PRIO
#define MLA_S_PRIO 3
#endif

static_assert(kSlotBytes % (1024 * kDmaWaves) == 0, "slot must split evenly over the waves");

#define MLA_VMCNT(n) (((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Row swizzle: logical 16-byte chunk `ch` of LDS row `t` sits at chunk position
// ch ^ swz(t), a permutation inside aligned groups of 8 chunks (a row has 72).
// LDS has 64 four-byte banks; a 1152-byte row moves the bank position by half
// of the 256-byte period, so row parity picks the half.  How gfx950 services a
// wave (measured with the SQ_LDS_BANK_CONFLICT counter): ds_read_b128 takes 16
// lanes per cycle, namely the lanes of one half-wave whose lane-index bits 2..4
// have equal parity; ds_read_b64_tr_b16 takes one half-wave per cycle.
// With swz(t) = 2 ((t >> 1) & 3):
//  * QK^T reads, lane 16g + q reading row q, chunk 4k + g: in one cycle
//    (q0, g0, q1 ^ g1, q2) takes all 16 values, so the 16 lanes hit 16
//    distinct bank groups;
//  * PV reads, row 4g + q/4, chunk 2c + q1, half q0: over a half-wave the
//    8-byte bank pair (q2, q1, q3 ^ c0, g0 ^ c1, q0) takes all 32 values.
__device__ __forceinline__ int swz(int t) { return ((t >> 1) & 3) << 1; }

// Maximum / sum over the four lanes q, q+16, q+32, q+48 (the 16-lane rows of
// a wave) with the gfx950 row-swap permutes: v_permlane16_swap exchanges rows
// 0<->1 and 2<->3 between its two operands, v_permlane32_swap the two halves.
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 16 bytes per lane from `base + voff` into LDS at m0 + 16 * lane.  (The
// instruction's immediate offset is left at 0: it would move the LDS
// destination as well.)
#ifndef MLA_DMA_POLICY
#define MLA_DMA_POLICY ""
#endif
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" MLA_DMA_POLICY ::"v"(voff), "s"(base), "{m0}"(lds_addr)
               : "memory");
}

// The same with the non-temporal bit.  At 16 heads every row is read by one
// workgroup and streams through once; the hint measured 35.7 -> 32.7 us on the
// V2-Lite workload.  (At 128 heads, where the two workgroups of an item read
// each row, it made no difference.)
__device__ __forceinline__ void dma16_nt(const char* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
}

// 4 bytes per lane from `base + voff` into LDS at m0 + 4 * lane: used only to
// pull rows into the L2 ahead of their DMA (the LDS bytes are never read).  No
// register receives the data, so nothing waits for it until the epilogue.
__device__ __forceinline__ void touch4(const char* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
}
// How many slices ahead of the one being scored the V waves without DMA pull
// rows into the L2 (0: off).  The four-slot LDS ring keeps only two slices in
// flight; these touches keep HBM reads of a third in flight as well.
#ifndef MLA_PREFETCH_D
#define MLA_PREFETCH_D 3
#endif

__device__ __forceinline__ bf16x8 lds_read128(const char* lds, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(lds + off);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const char* lds, uint32_t off) {
  short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)((__attribute__((address_space(3))) const char*)lds + off));
  return __builtin_bit_cast(bf16x4, v);
}

// ---------------------------------------------------------------------------
// H = 128, two workgroups per work item: workgroup half hh takes heads
// 64hh .. 64hh+63.  Both stream the same rows; the second read of a row is
// served by the L2 of the XCD they share (blocks i and i + 8 run on one XCD
// and are dispatched together).  Sixteen waves, four per SIMD, in two roles:
//  * S waves (w = 0..7): scores and softmax of head block hb = w % 4 (16
//    heads, Q fragments in 72 VGPRs) for token half th = w / 4 of every slice;
//  * V waves (w = 8..15): the latent PV of columns 64u .. 64u+63, u = w - 8,
//    for all 64 heads (64 accumulators); V waves u < 4 also run the DMA of
//    row group u.
// Iteration k: S waves score slice k and publish its weights; V waves
// accumulate slice k-1 with the weights published one iteration earlier.  One
// workgroup barrier per iteration (two in the first); the waves sharing a SIMD
// overlap their MFMA, LDS and VALU work.
//
// MFMA operand layouts (v_mfma_f32_16x16x32_bf16, lane l, g = l / 16, q = l % 16):
//   A[m][k]: lane holds m = q, k = 8g .. 8g+7;  B[k][n]: k = 8g .. 8g+7, n = q;
//   C[m][n]: lane holds m = 4g + i (i = 0..3), n = q.
// Scores: S^T[token][head], A = rows (token 16th + q, 8 latent values), B = Q^T.
// C leaves lane l with tokens 16th + 4g + i, head q.
// PV: O^T[latent][head] += C^T[latent][token] . P^T[token][head] with the
// reduction index k = 8g + j standing for token sigma(g, j) = 4g + j (j < 4) or
// 16 + 4g + (j - 4) (j >= 4): exactly the tokens whose weights lane l of the
// two S waves of a head block hold (token half 0 fills bytes 0..7 of the
// lane's 16-byte fragment, half 1 bytes 8..15).
// ---------------------------------------------------------------------------
constexpr int kHeadsWG = 64;
constexpr int kHeadBlocksWG = kHeadsWG / 16;        // 4
constexpr int kPBytesWG = kHeadBlocksWG * 64 * 16;  // 4 KiB of weights per slice
constexpr int kSWaves = 8;
static_assert(kStages * kSlotBytes + 2 * kPBytesWG + 256 + kSWaves * 4 + 4 * kHeadsWG * 4 + 4 <= 163840,
              "LDS budget");

__global__ __launch_bounds__(1024, 1) void decode_h128_kernel(
    const uint16_t* __restrict__ q_abs, const char* __restrict__ cache,
    const int32_t* __restrict__ block_table, int max_pages, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ items, int num_items, int q_len, float scale, float max_jump,
    float* __restrict__ o_part, float* __restrict__ lse_part, const int32_t* __restrict__ split_offsets,
    int32_t* __restrict__ tickets, float* __restrict__ o_latent, float* __restrict__ lse_out) {
  constexpr int H = 128;
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kSlotBytes + 2 * kPBytesWG];
  __shared__ __attribute__((aligned(16))) char junk[256];
  __shared__ int ticket_lds;
  __shared__ int votes[kSWaves];          // after a pass: jump flags of the S waves
  __shared__ float mref_x[2][kHeadsWG];   // per token half: a head's maximum
  __shared__ float lsum2[2][kHeadsWG];    // per token half: a head's row sum
  char* const pbuf = lds + kStages * kSlotBytes;
  const uint32_t lds_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;   // lane group (k block of the MFMA operands)
  const int q = lane & 15;   // row/column within a 16-block

  // block -> (item, query token, half): an item has per = 2 q_len workgroups;
  // blocks 8 per m + 8 r + j (j < 8, r < per) take part r of item 8m + j, so
  // all parts of an item run on one XCD (blocks go to XCDs round-robin) and
  // are dispatched together; a last incomplete group of items is laid out the
  // same way over the blocks that remain.  Part r = query token r / 2, half r % 2.
  int it, part;
  {
    const int per = 2 * q_len;
    const int blk = blockIdx.x;
    const int full = num_items & ~7;
    if (blk < per * full) {
      it = (blk / (8 * per)) * 8 + (blk & 7);
      part = (blk >> 3) % per;
    } else {
      const int j = blk - per * full, rest = num_items - full;
      it = full + j % rest;
      part = j / rest;
    }
  }
  const int hh = part & 1, tq = part >> 1;
  const int b = items[4 * it];
  const int p0 = items[4 * it + 2];
  const int p1 = items[4 * it + 3];
  const int L = seq_lens[b];
  const int t_begin = p0 * kPage;
  // query token tq sits at position L - q_len + tq and sees tokens up to it
  const int t_end = min(p1 * kPage, L - q_len + tq + 1);
  const int n_slices = (t_end - t_begin + kSliceTok - 1) / kSliceTok;
  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_pages;
  const int head0 = kHeadsWG * hh;
  const int64_t qrow0 = (static_cast<int64_t>(b) * q_len + tq) * H;    // q_abs row of head 0
  const int64_t prow0 = (static_cast<int64_t>(it) * q_len + tq) * H;   // partial row of head 0
  if (n_slices <= 0) {
    // none of the item's tokens is visible to this query token: an empty
    // partial (weight 0 in the merge); uniform over the workgroup, no barrier
    for (int i = threadIdx.x; i < kHeadsWG * kDc; i += blockDim.x)
      o_part[(prow0 + head0 + i / kDc) * kDc + i % kDc] = 0.f;
    if (threadIdx.x < kHeadsWG) lse_part[prow0 + head0 + threadIdx.x] = -INFINITY;
    return;
  }
  // Merged mode (tickets != null): o~ and lse of the sequence instead of a
  // partial when the sequence has one item, else the partial and, in the last
  // workgroup of the sequence half to finish, the merge of all its partials.
  const bool merged = tickets != nullptr;
  const int s0 = merged ? split_offsets[b] : 0;
  const int nsplit = merged ? split_offsets[b + 1] - s0 : 0;
  const bool direct = merged && nsplit == 1;
  const bool merge_tail = merged && nsplit > 1;

  auto slot_of = [&](int n) -> const char* { return lds + (n % kStages) * kSlotBytes; };
  auto pbuf_of = [&](int n) -> char* { return pbuf + (n & 1) * kPBytesWG; };

  // Slot layout: row t, logical chunk c at tile (t / 8, c / 8): (9 (t / 8) +
  // c / 8) KiB + 128 (t % 8) + 16 ((c % 8) ^ swz(t)); rows t and t + 16 are
  // kRowGroup2 bytes apart.
  constexpr uint32_t kTileRowGroup = 9 * 1024;
  constexpr uint32_t kRowGroup2 = 2 * kTileRowGroup;

  // Every wave runs the same sequence of workgroup barriers: a full pass has
  // n_slices + 4 of them, the exact-maximum pass n_slices + 2, the epilogue 1.
  if (w < kSWaves) {
    // ======================= S waves: scores and softmax =======================
    // The S waves are the critical path (their softmax cannot overlap their own
    // MFMAs); a higher issue priority lets the V waves' MFMAs fill the gaps.
    __builtin_amdgcn_s_setprio(MLA_S_PRIO);
    const int hb = w & 3, th = w >> 2;
    bf16x8 qf[18];  // B operand: head head0 + 16hb + q, values 32ks + 8g .. +8
    {
      const uint16_t* qrow = q_abs + (qrow0 + head0 + 16 * hb + q) * kDq + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
    }
    const int sw = swz(q);
    const uint32_t qk_base = th * kRowGroup2 + (q >> 3) * kTileRowGroup + (q & 7) * 128;
    const uint32_t qk_off0 = qk_base + 16 * ((g) ^ sw);      // even ks: logical chunk 8(ks/2) + g
    const uint32_t qk_off1 = qk_base + 16 * ((4 + g) ^ sw);  // odd ks: logical chunk 8(ks/2) + 4 + g
    const float c2 = scale * kLog2e;
    const int hidx = 16 * hb + q;  // head within the workgroup
    float m_ref = -INFINITY, l_run = 0.f;

    // S^T[16 tokens x 16 heads] of this token half, log2 units (scale folded
    // in); tokens of the slice at or past `nv` are -inf.  Two accumulator
    // chains (k parity), LDS reads kAhead steps ahead.
    auto scores = [&](const char* slot, int nv, float (&s)[4]) {
      float4_t acc[2] = {float4_t{0.f, 0.f, 0.f, 0.f}, float4_t{0.f, 0.f, 0.f, 0.f}};
      constexpr int kSteps = 18, kAhead = MLA_QK_AHEAD;
      auto off_of = [&](int ks) -> uint32_t {
        return 1024 * (ks >> 1) + ((ks & 1) ? qk_off1 : qk_off0);
      };
      bf16x8 fa[kAhead];
#pragma unroll
      for (int ks = 0; ks < kAhead; ++ks) fa[ks] = lds_read128(slot, off_of(ks));
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) {
        const bf16x8 a = fa[ks % kAhead];
        if (ks + kAhead < kSteps) fa[ks % kAhead] = lds_read128(slot, off_of(ks + kAhead));
        acc[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], acc[ks & 1], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = (acc[0][i] + acc[1][i]) * c2;
        s[i] = (16 * th + 4 * g + i < nv) ? v : -INFINITY;
      }
    };
    auto lane_max = [&](const float (&s)[4]) { return fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])); };
    auto nvalid = [&](int n) { return min(kSliceTok, t_end - (t_begin + n * kSliceTok)); };
    // weights 2^(s - m_ref) of slice k (masked tokens: 2^-inf = 0) into its buffer
    auto publish = [&](int k, const float (&s)[4]) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - m_ref);
      l_run += (p[0] + p[1]) + (p[2] + p[3]);
      const uint32_t pk[2] = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      *reinterpret_cast<bf16x4*>(pbuf_of(k) + (hb * 64 + lane) * 16 + 8 * th) =
          __builtin_bit_cast(bf16x4, pk);
    };

    // Full pass.  With `first`, m_ref is the per-head maximum of the first
    // slice (both token halves, exchanged through LDS) and the lane keeps a
    // running maximum of its later scores; the pass is discarded (returns
    // false) if some head's maximum exceeds m_ref by more than max_jump.
    // Slices 1 .. n-2 are whole, so only the first and the last are masked.
    auto full_pass = [&](bool first) -> bool {
      float m_lane = -INFINITY;
      float s[4];
      __syncthreads();
      scores(slot_of(0), nvalid(0), s);
      if (first) {
        const float m = rows_max(lane_max(s));
        if (g == 0) mref_x[th][hidx] = m;
      }
      __syncthreads();
      if (first) m_ref = fmaxf(mref_x[0][hidx], mref_x[1][hidx]);
      publish(0, s);
      for (int k = 1; k < n_slices - 1; ++k) {
        __syncthreads();
        scores(slot_of(k), kSliceTok, s);
        if (first) m_lane = fmaxf(m_lane, lane_max(s));
        publish(k, s);
      }
      if (n_slices > 1) {
        __syncthreads();
        scores(slot_of(n_slices - 1), nvalid(n_slices - 1), s);
        if (first) m_lane = fmaxf(m_lane, lane_max(s));
        publish(n_slices - 1, s);
      }
      __syncthreads();
      // vote: did a head of any S wave jump?
      const bool mine = __any(first && rows_max(m_lane) > m_ref + max_jump);
      if (lane == 0) votes[w] = mine ? 1 : 0;
      __syncthreads();
      int any = 0;
#pragma unroll
      for (int i = 0; i < kSWaves; ++i) any |= votes[i];
      __syncthreads();
      return any == 0;
    };

    if (!full_pass(true)) {
      // A head's maximum jumped by more than max_jump: exact maxima first,
      // then the item again against them (every weight <= 1).
      float m_lane = -INFINITY;
      for (int k = 0; k < n_slices; ++k) {
        __syncthreads();
        float s[4];
        scores(slot_of(k), nvalid(k), s);
        m_lane = fmaxf(m_lane, lane_max(s));
      }
      __syncthreads();
      const float m = rows_max(m_lane);
      if (g == 0) mref_x[th][hidx] = m;
      __syncthreads();
      m_ref = fmaxf(mref_x[0][hidx], mref_x[1][hidx]);
      l_run = 0.f;
      full_pass(false);
    }
    // epilogue: partial row sums to LDS, then the partial log-sum-exp
    const float l = rows_sum(l_run);
    if (g == 0) lsum2[th][hidx] = l;
    __syncthreads();
    if (th == 0 && g == 0) {
      const float lse_v = m_ref * kLn2 + logf(lsum2[0][hidx] + lsum2[1][hidx]);
      if (direct) {
        if (lse_out) lse_out[static_cast<int64_t>(b) * H + head0 + hidx] = lse_v;
      } else {
        lse_part[prow0 + head0 + hidx] = lse_v;
      }
    }
    if (merge_tail) {  // same barriers as the V waves' merge tail
      __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));  // this wave's stores have reached the L2
      __syncthreads();
      if (threadIdx.x == 0) {
        // release every wave's partial to the other XCDs (one L2 write-back),
        // then take the ticket
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        ticket_lds = atomicAdd(&tickets[2 * b + hh], 1);
      }
      __syncthreads();
      if (ticket_lds == nsplit - 1) {
        if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __syncthreads();
      }
    }
  } else {
    // ======================= V waves: DMA and latent PV =======================
    const int u = w - kSWaves;
    const bool dma = u < kDmaWaves;
    // DMA (u < 4): rows 8u .. 8u+7 of a slice, tiles j = 0..8 (tile (u, j) at
    // slot offset (9u + j) KiB).  Lane l covers row 8u + l/8 at chunk position
    // l % 8 of the tile, i.e. logical chunk 8j + ((l % 8) ^ swz(l / 8)).
    const int drow = 8 * u + (lane >> 3);
    const uint32_t dma_lane =
        static_cast<uint32_t>(drow * kRowBytes + ((lane & 7) ^ swz(lane >> 3)) * 16);
    auto issue = [&](int n) {
      const int tok0 = t_begin + n * kSliceTok;
      const int page = bt[tok0 >> 6];
      const char* src = cache + static_cast<int64_t>(page) * (kPage * kRowBytes) +
                        (tok0 & (kPage - 1)) * kRowBytes;
      const uint32_t dst = lds_base + (n % kStages) * kSlotBytes + kLoadsPerWave * u * 1024;
      // tail slice: rows of tokens >= nv are filled from token 0 of the slice
      // (finite data, weight 0), so empty cache slots are never read.
      const int nv = t_end - tok0;
      const uint32_t voff = drow < nv ? dma_lane : dma_lane - drow * kRowBytes;
#pragma unroll
      for (int j = 0; j < kLoadsPerWave; ++j) dma16(src + 128 * j, voff, dst + 1024 * j);
    };
    // L2 prefetch of slice n: the 288 128-byte lines of its 32 rows, the even
    // ones by half 0 of the pair and the odd ones by half 1 (the pair shares
    // the L2), one 4-byte load per line from the V waves without DMA
    const uint32_t junk_lds = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)junk));
    auto prefetch = [&](int n) {
      if (MLA_PREFETCH_D <= 0 || dma || n >= n_slices) return;
      const int tok0 = t_begin + n * kSliceTok;
      const int page = bt[tok0 >> 6];
      const char* src = cache + static_cast<int64_t>(page) * (kPage * kRowBytes) +
                        (tok0 & (kPage - 1)) * kRowBytes;
      const int nv = t_end - tok0;
      const int li = 2 * ((u - kDmaWaves) * 64 + lane) + hh;  // line of the slice
      if (li < 288 && li / 9 < nv) touch4(src, static_cast<uint32_t>(li * 128), junk_lds);
    };
    // wait for this wave's part of slice k (slice k+1 may stay in flight)
    auto wait_slice = [&](int k) {
      if (k + 1 < n_slices)
        __builtin_amdgcn_s_waitcnt(MLA_VMCNT(kLoadsPerWave));
      else
        __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
    };

    // PV A operand (transposed read): token 4g + q/4 (+16), column 16cb + 4(q%4)
    const int vrow = 4 * g + (q >> 2);
    const int vsw = swz(vrow);
    const uint32_t pv_base = (vrow >> 3) * kTileRowGroup + (vrow & 7) * 128 + 8 * (q & 1);
    const int pv_hc = (q & 3) >> 1;
    auto pv_off = [&](int cb) -> uint32_t {  // cb: global 16-column block 0..31
      return pv_base + 1024 * (cb >> 2) + 16 * ((2 * (cb & 3) + pv_hc) ^ vsw);
    };

    float4_t oacc[4][kHeadBlocksWG];  // [column block 4u + c][head block]
    auto zero_acc = [&]() {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int hb = 0; hb < kHeadBlocksWG; ++hb) oacc[c][hb] = float4_t{0.f, 0.f, 0.f, 0.f};
    };
    // O^T[64 columns x 64 heads] += C^T . P^T for one slice
    auto accumulate = [&](const char* slot, const char* pb) {
      bf16x8 pf[kHeadBlocksWG];
#pragma unroll
      for (int hb = 0; hb < kHeadBlocksWG; ++hb)
        pf[hb] = *reinterpret_cast<const bf16x8*>(pb + (hb * 64 + lane) * 16);
      bf16x4 f0[4], f1[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        f0[c] = lds_read_tr(slot, pv_off(4 * u + c));
        f1[c] = lds_read_tr(slot, pv_off(4 * u + c) + kRowGroup2);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 a = __builtin_shufflevector(f0[c], f1[c], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int hb = 0; hb < kHeadBlocksWG; ++hb)
          oacc[c][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[hb], oacc[c][hb], 0, 0, 0);
      }
    };
    auto full_pass = [&]() -> bool {
      if (dma) {
        issue(0);
        if (n_slices > 1) issue(1);
        wait_slice(0);
      }
      __syncthreads();
      if (dma && 2 < n_slices) issue(2);
      __syncthreads();  // the S waves' first-slice maximum exchange
      for (int n = 2; n <= MLA_PREFETCH_D; ++n) prefetch(n);
      for (int k = 1; k <= n_slices; ++k) {
        if (dma && k < n_slices) wait_slice(k);
        __syncthreads();
        if (dma && k + 2 < n_slices) issue(k + 2);
        prefetch(k + MLA_PREFETCH_D);
        accumulate(slot_of(k - 1), pbuf_of(k - 1));
      }
      // vote (written by the S waves)
      __syncthreads();
      int any = 0;
#pragma unroll
      for (int i = 0; i < kSWaves; ++i) any |= votes[i];
      __syncthreads();
      return any == 0;
    };

    zero_acc();
    if (!full_pass()) {
      // exact-maximum pass of the S waves: stream the slices again
      if (dma) {
        issue(0);
        if (n_slices > 1) issue(1);
      }
      for (int k = 0; k < n_slices; ++k) {
        if (dma) wait_slice(k);
        __syncthreads();
        if (dma && k + 2 < n_slices) issue(k + 2);
      }
      __syncthreads();
      __syncthreads();  // the S waves' maximum exchange
      zero_acc();
      full_pass();
    }
    // epilogue: normalise by the row sums of the S waves and write the partial
    // (or, for a sequence with one item in merged mode, o~ itself)
    if (MLA_PREFETCH_D > 0 && !dma) __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));  // prefetches landed
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < kHeadBlocksWG; ++hb) {
      const float inv = 1.f / (lsum2[0][16 * hb + q] + lsum2[1][16 * hb + q]);
      const int64_t row = direct ? static_cast<int64_t>(b) * H + head0 + 16 * hb + q
                                 : prow0 + head0 + 16 * hb + q;
      float* orow = (direct ? o_latent : o_part) + row * kDc + 64 * u + 4 * g;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        oacc[c][hb][0] *= inv;
        oacc[c][hb][1] *= inv;
        oacc[c][hb][2] *= inv;
        oacc[c][hb][3] *= inv;
        *reinterpret_cast<float4_t*>(orow + 16 * c) = oacc[c][hb];
      }
    }
    if (merge_tail) {
      // release this workgroup's partial, take a ticket (S wave 0 does both);
      // the last workgroup of the sequence half merges every partial in item
      // order (the combine's arithmetic, its own partial from registers) and
      // resets the ticket
      __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
      __syncthreads();
      __syncthreads();
      if (ticket_lds == nsplit - 1) {
        __syncthreads();  // after the acquire of S wave 0
#pragma unroll
        for (int hb = 0; hb < kHeadBlocksWG; ++hb) {
          const int head = head0 + 16 * hb + q;
          float M = -INFINITY;
          for (int s = s0; s < s0 + nsplit; ++s) M = fmaxf(M, lse_part[static_cast<int64_t>(s) * H + head]);
          float Z = 0.f;
          float4_t acc[4] = {};
          for (int s = s0; s < s0 + nsplit; ++s) {
            const int64_t r = static_cast<int64_t>(s) * H + head;
            const float wgt = expf(lse_part[r] - M);
            Z += wgt;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float4_t v = s == it ? oacc[c][hb]
                                         : *reinterpret_cast<const float4_t*>(o_part + r * kDc + 64 * u + 16 * c + 4 * g);
              acc[c][0] = fmaf(wgt, v[0], acc[c][0]);
              acc[c][1] = fmaf(wgt, v[1], acc[c][1]);
              acc[c][2] = fmaf(wgt, v[2], acc[c][2]);
              acc[c][3] = fmaf(wgt, v[3], acc[c][3]);
            }
          }
          const float inv = 1.f / Z;
          float* orow = o_latent + (static_cast<int64_t>(b) * H + head) * kDc + 64 * u + 4 * g;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[c][0] *= inv;
            acc[c][1] *= inv;
            acc[c][2] *= inv;
            acc[c][3] *= inv;
            *reinterpret_cast<float4_t*>(orow + 16 * c) = acc[c];
          }
          if (lse_out && u == 0 && g == 0) lse_out[static_cast<int64_t>(b) * H + head] = M + logf(Z);
        }
        if (u == 0 && lane == 0) tickets[2 * b + hh] = 0;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// H = 16: one workgroup of four waves per work item.  At 16 heads the step is
// far from the MFMA roof (about 30 flop per cached byte), so every wave
// computes the scores of all 16 heads over the whole slice itself: its score
// accumulators are then already the P^T operand of its own PV MFMAs (token
// order sigma(g, .), as above) and no weights cross between waves.  Wave w
// owns latent columns 128w .. 128w+127 of the PV (32 accumulators) and the DMA
// of row group w.  A ring of four slots keeps three slices in flight; the
// item's Q rows arrive through the fourth slot before the first slices.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 1) void decode_h16_kernel(
    const uint16_t* __restrict__ q_abs, const char* __restrict__ cache,
    const int32_t* __restrict__ block_table, int max_pages, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ items, int num_items, int q_len, float scale, float max_jump,
    float* __restrict__ o_part, float* __restrict__ lse_part, const int32_t* __restrict__ split_offsets,
    int32_t* __restrict__ tickets, float* __restrict__ o_latent, float* __restrict__ lse_out) {
  constexpr int H = 16;
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kSlotBytes];
  __shared__ int votes[4];
  __shared__ int ticket_lds;
  const uint32_t lds_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int q = lane & 15;

  // block -> (item, query token), laid out as in the 128-head kernel
  int it, tq;
  {
    const int blk = blockIdx.x;
    const int full = num_items & ~7;
    if (blk < q_len * full) {
      it = (blk / (8 * q_len)) * 8 + (blk & 7);
      tq = (blk >> 3) % q_len;
    } else {
      const int j = blk - q_len * full, rest = num_items - full;
      it = full + j % rest;
      tq = j / rest;
    }
  }
  const int b = items[4 * it];
  const int p0 = items[4 * it + 2];
  const int p1 = items[4 * it + 3];
  const int L = seq_lens[b];
  const int t_begin = p0 * kPage;
  const int t_end = min(p1 * kPage, L - q_len + tq + 1);
  const int n_slices = (t_end - t_begin + kSliceTok - 1) / kSliceTok;
  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_pages;
  const int64_t qrow0 = (static_cast<int64_t>(b) * q_len + tq) * H;
  const int64_t prow0 = (static_cast<int64_t>(it) * q_len + tq) * H;
  if (n_slices <= 0) {  // empty partial, as in the 128-head kernel
    for (int i = threadIdx.x; i < H * kDc; i += blockDim.x) o_part[prow0 * kDc + i] = 0.f;
    if (threadIdx.x < H) lse_part[prow0 + threadIdx.x] = -INFINITY;
    return;
  }
  constexpr uint32_t kTileRowGroup = 9 * 1024;
  constexpr uint32_t kRowGroup2 = 2 * kTileRowGroup;
  auto slot_of = [&](int n) -> const char* { return lds + (n % kStages) * kSlotBytes; };
  // merged mode, as in the 128-head kernel (one ticket per sequence)
  const bool merged = tickets != nullptr;
  const int s0 = merged ? split_offsets[b] : 0;
  const int nsplit = merged ? split_offsets[b + 1] - s0 : 0;
  const bool direct = merged && nsplit == 1;

  // Q fragments (B operand of the scores): head q, values 32ks + 8g .. +8
  // (staged through the LDS below, so that the first slices' DMA does not
  // wait for them)
  bf16x8 qf[18];

  // DMA: rows 8w .. 8w+7 of a slice (see the 128-head kernel)
  const int drow = 8 * w + (lane >> 3);
  const uint32_t dma_lane =
      static_cast<uint32_t>(drow * kRowBytes + ((lane & 7) ^ swz(lane >> 3)) * 16);
  auto issue = [&](int n) {
    const int tok0 = t_begin + n * kSliceTok;
    const int page = bt[tok0 >> 6];
    const char* src = cache + static_cast<int64_t>(page) * (kPage * kRowBytes) +
                      (tok0 & (kPage - 1)) * kRowBytes;
    const uint32_t dst = lds_base + (n % kStages) * kSlotBytes + kLoadsPerWave * w * 1024;
    const int nv = t_end - tok0;
    const uint32_t voff = drow < nv ? dma_lane : dma_lane - drow * kRowBytes;
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) dma16_nt(src + 128 * j, voff, dst + 1024 * j);
  };

  const int sw = swz(q);
  const uint32_t qk_base = (q >> 3) * kTileRowGroup + (q & 7) * 128;
  const uint32_t qk_off0 = qk_base + 16 * ((g) ^ sw);
  const uint32_t qk_off1 = qk_base + 16 * ((4 + g) ^ sw);
  const int vrow = 4 * g + (q >> 2);
  const int vsw = swz(vrow);
  const uint32_t pv_base = (vrow >> 3) * kTileRowGroup + (vrow & 7) * 128 + 8 * (q & 1);
  const int pv_hc = (q & 3) >> 1;
  auto pv_off = [&](int cb) -> uint32_t {
    return pv_base + 1024 * (cb >> 2) + 16 * ((2 * (cb & 3) + pv_hc) ^ vsw);
  };
  const float c2 = scale * kLog2e;

  // S^T[32 tokens x 16 heads], log2 units; tokens at or past `nv` are -inf
  auto scores = [&](const char* slot, int nv, float (&s)[2][4]) {
    float4_t acc[2][2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) acc[tb][0] = acc[tb][1] = float4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int kSteps = 36, kAhead = 8;
    auto off_of = [&](int st) -> uint32_t {
      const int ks = st >> 1, tb = st & 1;
      return tb * kRowGroup2 + 1024 * (ks >> 1) + ((ks & 1) ? qk_off1 : qk_off0);
    };
    bf16x8 fa[kAhead];
#pragma unroll
    for (int st = 0; st < kAhead; ++st) fa[st] = lds_read128(slot, off_of(st));
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int ks = st >> 1, tb = st & 1;
      const bf16x8 a = fa[st % kAhead];
      if (st + kAhead < kSteps) fa[st % kAhead] = lds_read128(slot, off_of(st + kAhead));
      acc[tb][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], acc[tb][ks & 1], 0, 0, 0);
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = (acc[tb][0][i] + acc[tb][1][i]) * c2;
        s[tb][i] = (tb * 16 + 4 * g + i < nv) ? v : -INFINITY;
      }
  };
  auto lane_max = [&](const float (&s)[2][4]) {
    return fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                 fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  };
  auto nvalid = [&](int n) { return min(kSliceTok, t_end - (t_begin + n * kSliceTok)); };

  float4_t oacc[8];
  float m_ref = -INFINITY, l_run = 0.f;
  // wait for slice n (later ones may stay in flight), then the ring barrier;
  // the slot of slice n-1 is free afterwards, so slice n+3 goes there
  auto enter = [&](int n) {
    const int ahead = min(kStages - 2, n_slices - 1 - n);
    if (ahead >= 2)
      __builtin_amdgcn_s_waitcnt(MLA_VMCNT(2 * kLoadsPerWave));
    else if (ahead == 1)
      __builtin_amdgcn_s_waitcnt(MLA_VMCNT(kLoadsPerWave));
    else
      __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
    __syncthreads();
    if (n + kStages - 1 < n_slices) issue(n + kStages - 1);
  };
  auto start = [&]() {
    for (int n = 0; n < kStages - 1 && n < n_slices; ++n) issue(n);
  };
  // weights and O += C^T P^T for one slice
  auto accumulate = [&](const char* slot, const float (&s)[2][4]) {
    float p[2][4];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[tb][i] = __builtin_amdgcn_exp2f(s[tb][i] - m_ref);
    l_run += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
    const uint32_t pk[4] = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                            pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pk);
    bf16x4 f0[8], f1[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      f0[c] = lds_read_tr(slot, pv_off(8 * w + c));
      f1[c] = lds_read_tr(slot, pv_off(8 * w + c) + kRowGroup2);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
      oacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_shufflevector(f0[c], f1[c], 0, 1, 2, 3, 4, 5, 6, 7), pf, oacc[c], 0, 0, 0);
  };

  // Full pass (see the softmax note at the top); every wave computes the same
  // scores, the vote only keeps the waves' control flow provably identical.
  auto full_pass = [&](bool first, bool started) -> bool {
#pragma unroll
    for (int c = 0; c < 8; ++c) oacc[c] = float4_t{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    float m_lane = -INFINITY;
    if (!started) start();
    for (int n = 0; n < n_slices; ++n) {
      enter(n);
      float s[2][4];
      scores(slot_of(n), nvalid(n), s);
      if (first) {
        if (n == 0)
          m_ref = rows_max(lane_max(s));
        else
          m_lane = fmaxf(m_lane, lane_max(s));
      }
      accumulate(slot_of(n), s);
    }
    const bool mine = __any(first && rows_max(m_lane) > m_ref + max_jump);
    __syncthreads();
    if (lane == 0) votes[w] = mine ? 1 : 0;
    __syncthreads();
    const bool any = (votes[0] | votes[1] | votes[2] | votes[3]) != 0;
    __syncthreads();
    return !any;
  };

  // The 16 Q rows of this item (18 KiB, contiguous in q_abs) go to ring slot 3
  // by DMA, ahead of the first three slices; slot 3 receives slice 3 only
  // after the barrier in enter(0), when every wave holds its fragments.
  {
    const char* qsrc = reinterpret_cast<const char*>(q_abs + qrow0 * kDq);
    const uint32_t qdst = lds_base + (kStages - 1) * kSlotBytes;
    for (int j = w; j < 18; j += 4) dma16(qsrc + 1024 * j, 16 * lane, qdst + 1024 * j);
  }
  start();
  // this wave's Q loads are done once only the slices' DMA may be outstanding
  switch (kLoadsPerWave * min(kStages - 1, n_slices)) {
    case 27: __builtin_amdgcn_s_waitcnt(MLA_VMCNT(27)); break;
    case 18: __builtin_amdgcn_s_waitcnt(MLA_VMCNT(18)); break;
    case 9: __builtin_amdgcn_s_waitcnt(MLA_VMCNT(9)); break;
    default: __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0)); break;
  }
  __syncthreads();
  {
    const char* qlds = lds + (kStages - 1) * kSlotBytes + q * kRowBytes + 16 * g;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qlds + 64 * ks);
  }

  if (!full_pass(true, true)) {
    float m_lane = -INFINITY;
    start();
    for (int n = 0; n < n_slices; ++n) {
      enter(n);
      float s[2][4];
      scores(slot_of(n), nvalid(n), s);
      m_lane = fmaxf(m_lane, lane_max(s));
    }
    __syncthreads();
    m_ref = rows_max(m_lane);
    full_pass(false, false);
  }

  const float l = rows_sum(l_run);
  if (w == 0 && g == 0) {
    const float lse_v = m_ref * kLn2 + logf(l);
    if (direct) {
      if (lse_out) lse_out[static_cast<int64_t>(b) * H + q] = lse_v;
    } else {
      lse_part[prow0 + q] = lse_v;
    }
  }
  const float inv = 1.f / l;
  float* orow = (direct ? o_latent + static_cast<int64_t>(b) * H * kDc
                        : o_part + prow0 * kDc) + q * kDc + 128 * w + 4 * g;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    oacc[c][0] *= inv;
    oacc[c][1] *= inv;
    oacc[c][2] *= inv;
    oacc[c][3] *= inv;
    *reinterpret_cast<float4_t*>(orow + 16 * c) = oacc[c];
  }
  if (merged && nsplit > 1) {
    __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));  // this wave's stores have reached the L2
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // one L2 write-back
      ticket_lds = atomicAdd(&tickets[2 * b], 1);
    }
    __syncthreads();
    if (ticket_lds == nsplit - 1) {
      if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __syncthreads();
      float M = -INFINITY;
      for (int s = s0; s < s0 + nsplit; ++s) M = fmaxf(M, lse_part[static_cast<int64_t>(s) * H + q]);
      float Z = 0.f;
      float4_t acc[8] = {};
      for (int s = s0; s < s0 + nsplit; ++s) {
        const int64_t r = static_cast<int64_t>(s) * H + q;
        const float wgt = expf(lse_part[r] - M);
        Z += wgt;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float4_t v = s == it ? oacc[c]
                                     : *reinterpret_cast<const float4_t*>(o_part + r * kDc + 128 * w + 16 * c + 4 * g);
          acc[c][0] = fmaf(wgt, v[0], acc[c][0]);
          acc[c][1] = fmaf(wgt, v[1], acc[c][1]);
          acc[c][2] = fmaf(wgt, v[2], acc[c][2]);
          acc[c][3] = fmaf(wgt, v[3], acc[c][3]);
        }
      }
      const float zinv = 1.f / Z;
      float* lrow = o_latent + (static_cast<int64_t>(b) * H + q) * kDc + 128 * w + 4 * g;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        acc[c][0] *= zinv;
        acc[c][1] *= zinv;
        acc[c][2] *= zinv;
        acc[c][3] *= zinv;
        *reinterpret_cast<float4_t*>(lrow + 16 * c) = acc[c];
      }
      if (lse_out && w == 0 && g == 0) lse_out[static_cast<int64_t>(b) * H + q] = M + logf(Z);
      if (threadIdx.x == 0) tickets[2 * b] = 0;
    }
  }
}

// Threshold (log2 units) beyond which a head's score maximum triggers the
// exact-maximum pass.  MLA_DECODE_MAX_JUMP overrides it (a value in (0, 30]),
// which lets tests drive that pass with ordinary inputs.
float max_jump() {
  const char* e = getenv("MLA_DECODE_MAX_JUMP");
  if (!e) return kMaxJumpDefault;
  const float v = strtof(e, nullptr);
  return (v > 0.f && v <= 30.f) ? v : kMaxJumpDefault;
}

}  // namespace

hipError_t decode_fast(const mla_dims& d, int q_len, const void* q_abs, const void* kv_cache,
                       const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                       const int32_t* items, int num_items, float* o_part, float* lse_part,
                       const int32_t* split_offsets, int32_t* tickets, float* o_latent,
                       float* lse_out, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(num_items) * q_len * (d.n_heads == 128 ? 2 : 1);
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (d.n_heads == 128) {
    hipLaunchKernelGGL(decode_h128_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(1024), 0, stream,
                       static_cast<const uint16_t*>(q_abs), static_cast<const char*>(kv_cache),
                       block_table, max_pages, seq_lens, items, num_items, q_len, d.softmax_scale,
                       max_jump(), o_part, lse_part, split_offsets, tickets, o_latent, lse_out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(decode_h16_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q_abs), static_cast<const char*>(kv_cache),
                     block_table, max_pages, seq_lens, items, num_items, q_len, d.softmax_scale,
                     max_jump(), o_part, lse_part, split_offsets, tickets, o_latent, lse_out);
  return hipGetLastError();
}

}  // namespace mla
