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
//  * Queries (128-head kernel): fetched once per workgroup by DMA into the two
//    ring slots that slices 2 and 3 later fill, then read into registers by
//    both S waves of a head block, so each CU takes them in once.
//  * QK^T operands: a lane reads 16 contiguous bytes (8 latent values of one
//    token) with ds_read_b128.
//  * PV operands: C^T needs 8 tokens of one latent column per lane; two
//    ds_read_b64_tr_b16 (4 tokens x 16 columns per 16-lane group, transposed
//    in the LDS crossbar) deliver them.  The MFMA's reduction index k is
//    permuted (k -> token sigma(g, k), see below) so that the QK^T
//    accumulators of a lane already hold the P^T operand of the same lane.
//
// Work split, every head count but 16 (decode_h128_kernel): ceil(H / 64)
// workgroups per work item, one per group of up to 64 heads (two at the
// 128 heads of V2, one per half), each with sixteen waves in two roles:
//  * eight S waves: scores of 16 heads over one 16-token half of every slice
//    (Q fragments stay in 72 VGPRs), turned into bf16 weights and put in a
//    4 KiB LDS exchange buffer;
//  * eight V waves: the latent PV of 64 columns for the workgroup's 64 heads
//    (64 accumulators), so each transposed C^T fragment feeds 4 MFMAs; four
//    of them also run the DMA, the other four the L2 prefetch.
//  The V waves run one slice behind the S waves; one workgroup barrier per
//  slice.  A last group with fewer than 64 heads runs its other head blocks
//  on zero queries and stores nothing of them.  H = 16 (decode_h16_kernel):
//  one workgroup of four waves per item, each scoring all 16 heads itself.
//
// Softmax in base 2 against a reference per head that starts at the maximum
// of the item's first slice and moves up to a later slice's maximum when that
// passes it by more than move_t (8 log2 units by default).  A move rescales
// the row sum and the accumulators of that head; between moves the
// accumulators are never touched.  Weights 2^(x - m_ref) above 1 are carried
// without loss of relative precision by the float32 accumulators and the bf16
// weights.
//  * H = 16: every wave computes the whole slice's scores, so it moves the
//    reference before it forms that slice's weights (weights <= 2^move_t).
//  * H = 128: the two token halves of a slice are scored by two S waves.  They
//    publish their maxima over each window of kMoveWindow slices, and both
//    take the same move when the next window starts (the V waves rescale
//    their accumulators before they add that window's first slice).  Inside a
//    window the weights can thus pass the reference by the window's own jump;
//    if that ever passes 2^safe_jump (64 by default) the workgroup agrees on
//    it through an LDS vote after the pass, takes the exact per-head maxima in
//    a scores-only pass and redoes the item against them.
// The result is the same softmax either way.
#include <math.h>
#include <stdlib.h>

#include <type_traits>

#include "decode_common.h"

namespace mla {
namespace {

using namespace dec;

constexpr int kStages = 4;
constexpr int kDmaWaves = 4;
constexpr int kLoadsPerWave = kSlotBytes / 1024 / kDmaWaves;  // 9 instructions of 1 KiB
// Work items the 128-head kernel redid against exact maxima since the count
// was last reset (per device; read and reset by exact_pass_count).
__device__ unsigned long long g_exact_passes = 0;

constexpr float kMoveDefault = 8.0f;       // log2 units: the reference moves past this
// The 128-head kernel decides reference moves once per window of this many
// slices (from the previous window's maxima).
#ifndef MLA_MOVE_WINDOW
#define MLA_MOVE_WINDOW 8
#endif
constexpr int kMoveWindow = MLA_MOVE_WINDOW;
static_assert(kMoveWindow >= 2 && (kMoveWindow & (kMoveWindow - 1)) == 0,
              "the loops find a window's last slice with a bit mask");
constexpr float kSafeJumpDefault = 64.0f;  // log2 units: an item is redone past this

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
// How many slices ahead of the one being scored the V waves without DMA pull
// rows into the L2 (0: off).  The four-slot LDS ring keeps only two slices in
// flight; these touches keep HBM reads of a third in flight as well.
#ifndef MLA_PREFETCH_D
#define MLA_PREFETCH_D 3
#endif

static_assert(kSlotBytes % (1024 * kDmaWaves) == 0, "slot must split evenly over the waves");

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
// LDS offset of the staged queries (18 steps x 4 head blocks x 1 KiB, ring
// slots 2 and 3)
constexpr uint32_t kQStageOff = 2 * kSlotBytes;
static_assert(18 * kHeadBlocksWG * 1024 == 2 * kSlotBytes, "the queries fill two ring slots");
static_assert(kStages * kSlotBytes + 2 * kPBytesWG + 256 + kSWaves * 4 + 4 * kHeadsWG * 4 +
                      2 * kHeadsWG * 4 + 2 * 4 * 4 + 2 * kHeadsWG * 4 + 4 <=
                  163840,
              "LDS budget");

__global__ __launch_bounds__(1024, 1) void decode_h128_kernel(
    const int32_t* __restrict__ items, const int32_t* __restrict__ order, int num_items, int q_len,
    int H, int max_pages, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ block_table, const char* __restrict__ cache,
    const uint16_t* __restrict__ q_abs, float scale, float move_t, float safe_jump,
    float* __restrict__ o_part, float* __restrict__ lse_part, const int32_t* __restrict__ split_offsets,
    int32_t* __restrict__ tickets, float* __restrict__ o_latent, float* __restrict__ lse_out) {
  // workgroups per item and query token, 64 heads each (the last one fewer
  // when 64 does not divide H)
  const int G = (H + kHeadsWG - 1) / kHeadsWG;
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kSlotBytes + 2 * kPBytesWG];
  __shared__ __attribute__((aligned(16))) char junk[256];
  __shared__ int ticket_lds;
  __shared__ int votes[kSWaves];          // after a pass: jump flags of the S waves
  __shared__ float mx_half[2][2][kHeadsWG];  // per window parity and token half: a head's maximum
  __shared__ float rsc[2][kHeadsWG];      // per window parity: a head's rescale factor
  __shared__ __attribute__((aligned(16))) int moved[2][kHeadBlocksWG];  // per window parity: slice of the last move
  __shared__ float lsum2[2][kHeadsWG];    // per token half: a head's row sum
  char* const pbuf = lds + kStages * kSlotBytes;
  const uint32_t lds_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;   // lane group (k block of the MFMA operands)
  const int q = lane & 15;   // row/column within a 16-block

  // block -> (item, part): an item has G q_len workgroups, all on one XCD and
  // dispatched together (block_to_item); part r = query token r / G, head
  // group r % G.
  int it, part;
  block_to_item(blockIdx.x, num_items, G * q_len, it, part);
  const int hh = part % G, tq = part / G;
  int b, p0, p1;
  load_item(items, order, it, b, p0, p1);  // dispatch slot -> item
  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_pages;
  const int page0 = first_page(bt, p0);  // slices 0 and 1 lie in page p0
  const int L = seq_lens[b];
  const int t_begin = p0 * kPage;
  // query token tq sits at position L - q_len + tq and sees tokens up to it
  const int t_end = min(p1 * kPage, L - q_len + tq + 1);
  const int n_slices = (t_end - t_begin + kSliceTok - 1) / kSliceTok;
  const int head0 = kHeadsWG * hh;
  // heads of this group: 64, or fewer in the last group when H is not a
  // multiple of 64 (a multiple of 16); the other head blocks run on zero
  // queries, so their weights are finite, and nothing of theirs is stored
  const int nh = min(kHeadsWG, H - head0);
  const int64_t qrow0 = (static_cast<int64_t>(b) * q_len + tq) * H;    // q_abs row of head 0
  const int64_t prow0 = (static_cast<int64_t>(it) * q_len + tq) * H;   // partial row of head 0
  if (n_slices <= 0) {
    // none of the item's tokens is visible to this query token: an empty
    // partial (weight 0 in the merge); uniform over the workgroup, no barrier
    for (int i = threadIdx.x; i < nh * kDc; i += blockDim.x)
      o_part[(prow0 + head0 + i / kDc) * kDc + i % kDc] = 0.f;
    if (threadIdx.x < nh) lse_part[prow0 + head0 + threadIdx.x] = -INFINITY;
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
  if (threadIdx.x < 2 * kHeadBlocksWG) (&moved[0][0])[threadIdx.x] = -2;

  // Slot layout: row t, logical chunk c at tile (t / 8, c / 8): (9 (t / 8) +
  // c / 8) KiB + 128 (t % 8) + 16 ((c % 8) ^ swz(t)); rows t and t + 16 are
  // kRowGroup2 bytes apart.

  // Every wave runs the same sequence of workgroup barriers: a full pass has
  // n_slices + 4 of them, the exact-maximum pass n_slices + 2, the epilogue 1.
  if (w < kSWaves) {
    // ======================= S waves: scores and softmax =======================
    // The S waves are the critical path (their softmax cannot overlap their own
    // MFMAs); a higher issue priority lets the V waves' MFMAs fill the gaps.
    __builtin_amdgcn_s_setprio(MLA_S_PRIO);
    const int hb = w & 3, th = w >> 2;
    bf16x8 qf[18];  // B operand: head head0 + 16hb + q, values 32ks + 8g .. +8
    // The queries reach the CU once, by DMA into ring slots 2 and 3 (free
    // until slice 2 is issued), instead of once per token half: 1 KiB block
    // (ks, hb) holds at lane position 16g + q the operand of lane 16g + q.
    // Token half th fetches steps 9th .. 9th + 8 of its head block; after the
    // barrier both halves read all 18.
    const uint32_t q_lds = kQStageOff + 1024 * hb;
    if (16 * hb < nh) {
      const char* qsrc = reinterpret_cast<const char*>(q_abs + (qrow0 + head0 + 16 * hb) * kDq);
      const uint32_t qoff = static_cast<uint32_t>(q * kRowBytes + 16 * g);
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        const int ks = 9 * th + j;
        dma16(qsrc + 64 * ks, qoff, lds_base + q_lds + 4096 * ks);
      }
      __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
    }
    __syncthreads();  // every query block is in the LDS
    if (16 * hb < nh) {
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qf[ks] = lds_read128(lds, q_lds + 4096 * ks + 16 * lane);
    } else {
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qf[ks] = bf16x8{};
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

    // Reference moves, once per window of kMoveWindow slices.  At the end of
    // window v the S waves publish their half's per-head maximum over the
    // window (mx_half[v & 1]); when window v + 1 starts (slice k =
    // kMoveWindow (v + 1)), both S waves of a head block read the two values,
    // and heads whose window maximum passed m_ref + move_t move their
    // reference there, before slice k's weights are formed.  The two waves
    // see the same values and so take the same decision.  The row sum is
    // rescaled at once; the V waves rescale the accumulators of that head
    // block before they add slice k (the factor and the slice index of the
    // move go through LDS).
    auto move_ref = [&](int k, float mprev) {
      const bool up = mprev > m_ref + move_t;
      if (__any(up)) {
        const float m_new = up ? mprev : m_ref;
        const float r = __builtin_amdgcn_exp2f(m_ref - m_new);
        l_run *= r;
        m_ref = m_new;
        const int v = k / kMoveWindow;
        if (th == 0) {
          if (g == 0) rsc[v & 1][hidx] = r;
          if (lane == 0) moved[v & 1][hb] = k;
        }
      }
    };

    // Full pass.  With `first`, m_ref starts at the per-head maximum of the
    // first slice (both token halves, exchanged through LDS) and moves up
    // during the pass (move_ref); a weight can thus exceed 1 by the jump of
    // the scores within one window.  The pass is discarded (returns false) if
    // that ever passes 2^safe_jump.  Without `first`, m_ref holds the exact
    // maxima and does not move.
    auto full_pass = [&](bool first) -> bool {
      float e_lane = -INFINITY;  // largest weight exponent s - m_ref published
      float m_win = -INFINITY;   // this lane's maximum over the current window
      float s[4];
      __syncthreads();
      scores(slot_of(0), nvalid(0), s);
      if (first) {
        const float m = rows_max(lane_max(s));
        if (g == 0) mx_half[0][th][hidx] = m;
      }
      __syncthreads();
      if (first) m_ref = fmaxf(mx_half[0][0][hidx], mx_half[0][1][hidx]);
      publish(0, s);
      // slice k (k >= 1) holds nv valid tokens; with the window work of a
      // window's first slice (move test) and last slice (its maxima).
      // edge_c: 1 for a window's first slice, 2 for its last, 0 to test k.
      auto step = [&](int k, int nv, auto edge_c) {
        constexpr int edge = decltype(edge_c)::value;
        __syncthreads();
        const bool check = first && (edge == 1 || (edge == 0 && k % kMoveWindow == 0));
        const bool wend = edge == 2 || (edge == 0 && k % kMoveWindow == kMoveWindow - 1);
        float mp0 = -INFINITY, mp1 = -INFINITY;
        if (check) {  // the previous window's maxima, read before the MFMAs
          const int v = k / kMoveWindow - 1;
          mp0 = mx_half[v & 1][0][hidx];
          mp1 = mx_half[v & 1][1][hidx];
        }
        scores(slot_of(k), nv, s);
        if (first) {
          if (check) move_ref(k, fmaxf(mp0, mp1));
          m_win = fmaxf(m_win, lane_max(s));
          if (wend) {  // window k / kMoveWindow ends
            // m_ref is constant within a window: its weights' largest exponent
            e_lane = fmaxf(e_lane, m_win - m_ref);
            const float mh = rows_max(m_win);  // every lane takes part in the row permutes
            if (g == 0) mx_half[(k / kMoveWindow) & 1][th][hidx] = mh;
            m_win = -INFINITY;
          }
        }
        publish(k, s);
      };
      // a whole slice that is neither the first nor the last of its window
      // (no window work: its branches cost the critical path on every slice)
      auto step_inner = [&](int k) {
        __syncthreads();
        scores(slot_of(k), kSliceTok, s);
        if (first) m_win = fmaxf(m_win, lane_max(s));
        publish(k, s);
      };
      // slices 1 .. n-2 are whole (the constant count lets the compiler drop
      // the mask); only the first and the last can be short.  Per window: its
      // first slice, the inner slices, its last slice (window 0 starts at 1).
      using First = std::integral_constant<int, 1>;
      using Last = std::integral_constant<int, 2>;
      int k = 1;
      for (const int e = min(n_slices - 1, kMoveWindow - 1); k < e; ++k) step_inner(k);
      if (k < n_slices - 1) step(k++, kSliceTok, Last{});
      while (k < n_slices - 1) {  // k starts a window
        step(k++, kSliceTok, First{});
        for (const int e = min(n_slices - 1, k | (kMoveWindow - 1)); k < e; ++k) step_inner(k);
        if (k < n_slices - 1) step(k++, kSliceTok, Last{});
      }
      if (n_slices > 1) step(n_slices - 1, nvalid(n_slices - 1), std::integral_constant<int, 0>{});
      e_lane = fmaxf(e_lane, m_win - m_ref);  // a last, partial window
      __syncthreads();
      // vote: did a weight of any S wave pass 2^safe_jump?
      const bool mine = __any(first && e_lane > safe_jump);
      if (lane == 0) votes[w] = mine ? 1 : 0;
      __syncthreads();
      int any = 0;
#pragma unroll
      for (int i = 0; i < kSWaves; ++i) any |= votes[i];
      __syncthreads();
      return any == 0;
    };

    if (!full_pass(true)) {
      // A weight passed 2^safe_jump (one slice jumped that far past the
      // reference): exact maxima first, then the item again against them
      // (every weight <= 1, no moves).
      if (threadIdx.x == 0) atomicAdd(&g_exact_passes, 1ull);
      float m_lane = -INFINITY;
      for (int k = 0; k < n_slices; ++k) {
        __syncthreads();
        float s[4];
        scores(slot_of(k), nvalid(k), s);
        m_lane = fmaxf(m_lane, lane_max(s));
      }
      __syncthreads();
      const float m = rows_max(m_lane);
      if (g == 0) mx_half[0][th][hidx] = m;
      __syncthreads();
      m_ref = fmaxf(mx_half[0][0][hidx], mx_half[0][1][hidx]);
      l_run = 0.f;
      full_pass(false);
    }
    // epilogue: partial row sums to LDS, then the partial log-sum-exp
    const float l = rows_sum(l_run);
    if (g == 0) lsum2[th][hidx] = l;
    __syncthreads();
    if (th == 0 && g == 0 && hidx < nh) {
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
        ticket_lds = atomicAdd(&tickets[G * b + hh], 1);
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
      const int page = n < 2 ? page0 : bt[tok0 >> 6];
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
    // L2 prefetch of slice n: the 288 128-byte lines of its 32 rows, line i by
    // head group i mod G (at 128 heads the even lines by one half of the pair
    // and the odd ones by the other: the item's workgroups share the L2), one
    // 4-byte load per line from the V waves without DMA
    const uint32_t junk_lds = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)junk));
    auto prefetch = [&](int n) {
      if (MLA_PREFETCH_D <= 0 || dma || n >= n_slices) return;
      const int tok0 = t_begin + n * kSliceTok;
      const int page = bt[tok0 >> 6];
      const char* src = cache + static_cast<int64_t>(page) * (kPage * kRowBytes) +
                        (tok0 & (kPage - 1)) * kRowBytes;
      const int nv = t_end - tok0;
      for (int li = G * ((u - kDmaWaves) * 64 + lane) + hh; li < 288 && li / 9 < nv; li += G * 256)
        touch4(src, static_cast<uint32_t>(li * 128), junk_lds);  // line li of the slice
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
    // O^T[64 columns x 64 heads] += C^T . P^T for slice k; with `moves`, first
    // the rescale of the head blocks whose reference moved at slice k
    // (may_move_c: std::true_type for a slice that can start a window, else
    // std::false_type, which leaves out the move test altogether)
    // C^T fragments of the slice to accumulate next, read at the end of the
    // iteration before (slice k is in the LDS from barrier k on, and its slot
    // is refilled two iterations later), so that after a barrier the V waves
    // read only the weights before their MFMAs
    bf16x4 fc0[4], fc1[4];
    auto read_ct = [&](int k) {
      const char* slot = slot_of(k);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        fc0[c] = lds_read_tr(slot, pv_off(4 * u + c));
        fc1[c] = lds_read_tr(slot, pv_off(4 * u + c) + kRowGroup2);
      }
    };
    // slice k with the C^T fragments in fc0/fc1; then the next slice's
    // fragments when `next` (in flight across the barrier, used next
    // iteration)
    auto accumulate = [&](int k, bool moves, auto may_move_c, bool next) {
      constexpr bool may_move = decltype(may_move_c)::value;
      const char* pb = pbuf_of(k);
      // the slice indices of the last moves first (at window starts), then
      // every operand read of the slice; the scheduling barrier keeps that
      // order, so the move test waits only for its own read
      moves = may_move && moves && k > 0 && k % kMoveWindow == 0;  // moves happen at window starts only
      int4 mv = {-1, -1, -1, -1};
      if (moves) mv = *reinterpret_cast<const int4*>(&moved[(k / kMoveWindow) & 1][0]);
      bf16x8 pf[kHeadBlocksWG];
#pragma unroll
      for (int hb = 0; hb < kHeadBlocksWG; ++hb)
        pf[hb] = *reinterpret_cast<const bf16x8*>(pb + (hb * 64 + lane) * 16);
      if (may_move) __builtin_amdgcn_sched_barrier(0);
      if (moves) {
        const int hit = (__builtin_amdgcn_readfirstlane(mv.x) == k ? 1 : 0) |
                        (__builtin_amdgcn_readfirstlane(mv.y) == k ? 2 : 0) |
                        (__builtin_amdgcn_readfirstlane(mv.z) == k ? 4 : 0) |
                        (__builtin_amdgcn_readfirstlane(mv.w) == k ? 8 : 0);
        if (hit) {
          // whole-vector products, written out per head block: indexed element
          // updates in a loop kept the compiler from holding oacc in registers
          static_assert(kHeadBlocksWG == 4, "one line per head block below");
          const int v = (k / kMoveWindow) & 1;
          const float r0 = (hit & 1) ? rsc[v][q] : 1.f;
          const float r1 = (hit & 2) ? rsc[v][16 + q] : 1.f;
          const float r2 = (hit & 4) ? rsc[v][32 + q] : 1.f;
          const float r3 = (hit & 8) ? rsc[v][48 + q] : 1.f;
          oacc[0][0] *= r0; oacc[1][0] *= r0; oacc[2][0] *= r0; oacc[3][0] *= r0;
          oacc[0][1] *= r1; oacc[1][1] *= r1; oacc[2][1] *= r1; oacc[3][1] *= r1;
          oacc[0][2] *= r2; oacc[1][2] *= r2; oacc[2][2] *= r2; oacc[3][2] *= r2;
          oacc[0][3] *= r3; oacc[1][3] *= r3; oacc[2][3] *= r3; oacc[3][3] *= r3;
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 a = __builtin_shufflevector(fc0[c], fc1[c], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int hb = 0; hb < kHeadBlocksWG; ++hb)
          oacc[c][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[hb], oacc[c][hb], 0, 0, 0);
      }
      if (next) read_ct(k + 1);
    };
    // `issued`: slices 0 and 1 are already in flight
    auto full_pass = [&](bool first, bool issued) -> bool {
      if (dma) {
        if (!issued) {
          issue(0);
          if (n_slices > 1) issue(1);
        }
        wait_slice(0);
      }
      __syncthreads();
      if (dma && 2 < n_slices) issue(2);
      read_ct(0);
      __syncthreads();  // the S waves' first-slice maximum exchange
      for (int n = 2; n <= MLA_PREFETCH_D; ++n) prefetch(n);
      // iteration k adds slice k - 1; only a slice that starts a window
      // (k - 1 a multiple of kMoveWindow) carries the move test
      auto vstep = [&](int k, auto may_move_c) {
        if (dma && k < n_slices) wait_slice(k);
        __syncthreads();
        if (dma && k + 2 < n_slices) issue(k + 2);
        prefetch(k + MLA_PREFETCH_D);
        accumulate(k - 1, first, may_move_c, k < n_slices);
      };
      for (int k = 1; k <= n_slices;) {
        vstep(k++, std::true_type{});
        const int next = (k - 1 + kMoveWindow - 1) / kMoveWindow * kMoveWindow + 1;  // next window start
        for (const int e = min(n_slices + 1, next); k < e; ++k) vstep(k, std::false_type{});
      }
      // vote (written by the S waves)
      __syncthreads();
      int any = 0;
#pragma unroll
      for (int i = 0; i < kSWaves; ++i) any |= votes[i];
      __syncthreads();
      return any == 0;
    };

    // the first slices go out beside the S waves' query DMA
    if (dma) {
      issue(0);
      if (n_slices > 1) issue(1);
    }
    __syncthreads();  // the queries are in the LDS (the S waves' first barrier)
    zero_acc();
    if (!full_pass(true, true)) {
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
      full_pass(false, false);
    }
    // epilogue: normalise by the row sums of the S waves and write the partial
    // (or, for a sequence with one item in merged mode, o~ itself)
    if (MLA_PREFETCH_D > 0 && !dma) __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));  // prefetches landed
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < kHeadBlocksWG; ++hb) {
      if (16 * hb >= nh) continue;  // a head block past H (uniform over the wave)
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
        if (u == 0 && lane == 0) tickets[G * b + hh] = 0;
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
    const int32_t* __restrict__ items, const int32_t* __restrict__ order, int num_items, int q_len,
    int H, int max_pages, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ block_table, const char* __restrict__ cache,
    const uint16_t* __restrict__ q_abs, float scale, float move_t, float safe_jump,
    float* __restrict__ o_part, float* __restrict__ lse_part, const int32_t* __restrict__ split_offsets,
    int32_t* __restrict__ tickets, float* __restrict__ o_latent, float* __restrict__ lse_out) {
  const int G = H / 16;  // workgroups per item and query token (the launch uses this kernel at 16 heads: one)
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kSlotBytes];
  __shared__ int ticket_lds;
  const uint32_t lds_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int q = lane & 15;

  // block -> (item, query token), laid out as in the 128-head kernel
  int it, part;
  block_to_item(blockIdx.x, num_items, G * q_len, it, part);
  const int head0 = 16 * (part % G), tq = part / G;
  int b, p0, p1;
  load_item(items, order, it, b, p0, p1);  // dispatch slot -> item
  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_pages;
  const int page0 = first_page(bt, p0);  // slices 0 and 1 lie in page p0
  const int L = seq_lens[b];
  const int t_begin = p0 * kPage;
  const int t_end = min(p1 * kPage, L - q_len + tq + 1);
  const int n_slices = (t_end - t_begin + kSliceTok - 1) / kSliceTok;
  const int64_t qrow0 = (static_cast<int64_t>(b) * q_len + tq) * H + head0;  // q_abs row of the first head
  const int64_t prow0 = (static_cast<int64_t>(it) * q_len + tq) * H + head0;  // its partial row
  if (n_slices <= 0) {  // empty partial, as in the 64-head kernel
    for (int i = threadIdx.x; i < 16 * kDc; i += blockDim.x) o_part[prow0 * kDc + i] = 0.f;
    if (threadIdx.x < 16) lse_part[prow0 + threadIdx.x] = -INFINITY;
    return;
  }
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
    const int page = n < 2 ? page0 : bt[tok0 >> 6];
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

  // The pass.  Every wave computes the same scores (the same operands in the
  // same order), so every wave takes the same softmax decisions: the
  // reference starts at the first slice's per-head maximum and moves up to a
  // slice's maximum, before that slice's weights are formed, when the maximum
  // passes it by more than move_t.  A move rescales the wave's own
  // accumulators and row sum; weights never exceed 2^move_t.
  auto full_pass = [&]() {
#pragma unroll
    for (int c = 0; c < 8; ++c) oacc[c] = float4_t{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    for (int n = 0; n < n_slices; ++n) {
      enter(n);
      float s[2][4];
      scores(slot_of(n), nvalid(n), s);
      const float mx = rows_max(lane_max(s));
      if (n == 0) {
        m_ref = mx;
      } else {
        const bool up = mx > m_ref + move_t;
        if (__any(up)) {
          const float m_new = up ? mx : m_ref;
          const float r = __builtin_amdgcn_exp2f(m_ref - m_new);
          l_run *= r;
          // whole-vector products, written out: indexed element updates inside
          // the branch kept the compiler from holding oacc in registers
          oacc[0] *= r;
          oacc[1] *= r;
          oacc[2] *= r;
          oacc[3] *= r;
          oacc[4] *= r;
          oacc[5] *= r;
          oacc[6] *= r;
          oacc[7] *= r;
          m_ref = m_new;
        }
      }
      accumulate(slot_of(n), s);
    }
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

  full_pass();

  const float l = rows_sum(l_run);
  if (w == 0 && g == 0) {
    const float lse_v = m_ref * kLn2 + logf(l);
    if (direct) {
      if (lse_out) lse_out[static_cast<int64_t>(b) * H + head0 + q] = lse_v;
    } else {
      lse_part[prow0 + q] = lse_v;
    }
  }
  const float inv = 1.f / l;
  float* orow = (direct ? o_latent + (static_cast<int64_t>(b) * H + head0) * kDc
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
      for (int s = s0; s < s0 + nsplit; ++s) M = fmaxf(M, lse_part[static_cast<int64_t>(s) * H + head0 + q]);
      float Z = 0.f;
      float4_t acc[8] = {};
      for (int s = s0; s < s0 + nsplit; ++s) {
        const int64_t r = static_cast<int64_t>(s) * H + head0 + q;
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
      float* lrow = o_latent + (static_cast<int64_t>(b) * H + head0 + q) * kDc + 128 * w + 4 * g;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        acc[c][0] *= zinv;
        acc[c][1] *= zinv;
        acc[c][2] *= zinv;
        acc[c][3] *= zinv;
        *reinterpret_cast<float4_t*>(lrow + 16 * c) = acc[c];
      }
      if (lse_out && w == 0 && g == 0) lse_out[static_cast<int64_t>(b) * H + head0 + q] = M + logf(Z);
      if (threadIdx.x == 0) tickets[2 * b] = 0;
    }
  }
}

// Reference-move threshold (log2 units).  MLA_DECODE_MAX_JUMP overrides it (a
// value in (0, 30]); tests use a small value to move the reference on
// ordinary inputs.
float move_threshold() {
  const char* e = getenv("MLA_DECODE_MAX_JUMP");
  if (!e) return kMoveDefault;
  const float v = strtof(e, nullptr);
  return (v > 0.f && v <= 30.f) ? v : kMoveDefault;
}

// Largest weight exponent (log2 units past the reference) the 128-head kernel
// keeps before it redoes an item against exact maxima.  MLA_DECODE_SAFE_JUMP
// overrides it (a value in (0, 100]); tests use a small value to drive that
// pass with ordinary inputs.
float safe_jump() {
  const char* e = getenv("MLA_DECODE_SAFE_JUMP");
  if (!e) return kSafeJumpDefault;
  const float v = strtof(e, nullptr);
  return (v > 0.f && v <= 100.f) ? v : kSafeJumpDefault;
}

}  // namespace

hipError_t exact_pass_count(uint64_t* count, bool reset) {
  unsigned long long v = 0;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_exact_passes), sizeof(v));
  if (e != hipSuccess) return e;
  if (reset) {
    const unsigned long long zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_exact_passes), &zero, sizeof(zero));
    if (e != hipSuccess) return e;
  }
  *count = v;
  return hipSuccess;
}

hipError_t decode_fast(const mla_dims& d, int q_len, const void* q_abs, const void* kv_cache,
                       const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                       const int32_t* items, int num_items, const int32_t* order, float* o_part,
                       float* lse_part,
                       const int32_t* split_offsets, int32_t* tickets, float* o_latent,
                       float* lse_out, hipStream_t stream) {
  // 16 heads take the 16-heads-per-workgroup kernel; every other multiple of
  // 16 takes ceil(H / 64) workgroups of 64 heads per item (the last one
  // partly on zero queries when 64 does not divide H): with one workgroup
  // per 64 heads each row is taken in by as few CUs as possible
  const bool wide = d.n_heads != 16;
  const int groups = wide ? (d.n_heads + kHeadsWG - 1) / kHeadsWG : 1;
  const int64_t blocks = static_cast<int64_t>(num_items) * q_len * groups;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (wide) {
    hipLaunchKernelGGL(decode_h128_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(1024), 0, stream,
                       items, order, num_items, q_len, d.n_heads, max_pages, seq_lens, block_table,
                       static_cast<const char*>(kv_cache), static_cast<const uint16_t*>(q_abs),
                       d.softmax_scale, move_threshold(), safe_jump(), o_part, lse_part, split_offsets,
                       tickets, o_latent, lse_out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(decode_h16_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     items, order, num_items, q_len, d.n_heads, max_pages, seq_lens, block_table,
                     static_cast<const char*>(kv_cache), static_cast<const uint16_t*>(q_abs),
                     d.softmax_scale, move_threshold(), safe_jump(), o_part, lse_part, split_offsets,
                     tickets, o_latent, lse_out);
  return hipGetLastError();
}

}  // namespace mla
