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
//    no VGPR round trip) into a ring of 32-token slots (36,864 bytes each).
//    The 16-byte chunk `ch` of token row `t` sits at chunk position
//    ch ^ swz(t) of that row in LDS, which keeps both read patterns below free
//    of bank conflicts.  Each lane picks which global chunk it fetches, so the
//    swizzle costs nothing at load time.
//  * QK^T operands: a lane reads 16 contiguous bytes (8 latent values of one
//    token) with ds_read_b128.
//  * PV operands: C^T needs 8 tokens of one latent column per lane; two
//    ds_read_b64_tr_b16 (4 tokens x 16 columns per 16-lane group, transposed
//    in the LDS crossbar) deliver them.  The MFMA's reduction index k is
//    permuted (k -> token sigma(g, k)) so that P^T comes straight out of the
//    S^T accumulators of the same lanes with no shuffle.
//  * One workgroup barrier per slice protects the ring.
//
// Work split inside a workgroup (4 waves, one per SIMD):
//  * H = 128: wave w owns heads 32w .. 32w+31 over every token of the item
//    (Q fragments: 144 VGPRs; O^T accumulators: 256 registers).
// Softmax in base 2 against a fixed reference per head: the maximum of the
// item's first slice.  Weights 2^(x - m_ref) may exceed 1 by up to 2^20, which
// float32 accumulators and bf16 weights carry without loss of relative
// precision, so the 256 accumulators are never rescaled in registers.  If a
// later slice exceeds the reference by more than 2^20, the workgroup agrees on
// it through an LDS flag at the next barrier, takes the exact per-head maxima in
// a scores-only pass and redoes the item against them; the result is the same
// softmax either way.
#include <math.h>
#include <stdlib.h>

#include <type_traits>

#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kRowBytes = kDq * 2;             // 1152
constexpr int kChunksPerRow = kRowBytes / 16;  // 72
constexpr int kSliceTok = 32;
constexpr int kSlotBytes = kSliceTok * kRowBytes;  // 36,864
constexpr int kStages = 4;
constexpr int kWaves = 4;
constexpr int kLoadsPerWave = kSlotBytes / 1024 / kWaves;  // 9 instructions of 1 KiB
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMaxJumpDefault = 20.0f;  // log2 units; see the softmax note above

static_assert(kSlotBytes % (1024 * kWaves) == 0, "slot must split evenly over the waves");

#define MLA_VMCNT(n) (((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Row swizzle: chunk position of logical chunk `ch` in LDS row `t` is ch ^ swz(t).
// For 8 consecutive rows (QK^T reads) and for 4 consecutive rows x 2 adjacent
// chunks (PV transposed reads) the positions land in distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// 16 bytes per lane from `base + voff` into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr)
               : "memory");
}

__device__ __forceinline__ bf16x8 lds_read128(const char* lds, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(lds + off);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const char* lds, uint32_t off) {
  short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)((__attribute__((address_space(3))) const char*)lds + off));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16_bits(a)) |
         (static_cast<uint32_t>(f32_to_bf16_bits(b)) << 16);
}

// ---------------------------------------------------------------------------
// H = 128: head split.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 1) void decode_h128_kernel(
    const uint16_t* __restrict__ q_abs, const char* __restrict__ cache,
    const int32_t* __restrict__ block_table, int max_pages, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ items, float scale, float max_jump, float* __restrict__ o_part,
    float* __restrict__ lse_part) {
  constexpr int H = 128;
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kSlotBytes];
  const uint32_t lds_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;   // lane group (k block of the MFMA operands)
  const int q = lane & 15;   // row/column within a 16-block

  const int it = blockIdx.x;
  const int b = items[4 * it];
  const int p0 = items[4 * it + 2];
  const int p1 = items[4 * it + 3];
  const int L = seq_lens[b];
  const int t_begin = p0 * kPage;
  const int t_end = min(p1 * kPage, L);
  const int n_slices = (t_end - t_begin + kSliceTok - 1) / kSliceTok;
  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_pages;

  // --- Q fragments (B operand of S^T = Rows . Q^T): lane holds head q of
  // block hb, values 32ks + 8g .. +8.
  bf16x8 qf[2][18];
  {
    const uint16_t* qrow0 = q_abs + (static_cast<int64_t>(b) * H + 32 * w + q) * kDq + 8 * g;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int ks = 0; ks < 18; ++ks)
        qf[hb][ks] = *reinterpret_cast<const bf16x8*>(qrow0 + hb * 16 * kDq + 32 * ks);
  }
  __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));

  // --- per-lane DMA source: LDS chunk p = (9w + i) * 64 + lane of a slot holds
  // logical chunk ch = (p % 72) ^ swz(t) of token t = p / 72.
  auto dma_token = [&](int i) { return ((kLoadsPerWave * w + i) * 64 + lane) / kChunksPerRow; };
  auto dma_off = [&](int i) -> uint32_t {
    const int p = (kLoadsPerWave * w + i) * 64 + lane;
    const int t = p / kChunksPerRow;
    return static_cast<uint32_t>(t * kRowBytes + ((p % kChunksPerRow) ^ swz(t)) * 16);
  };

  auto issue = [&](int n) {
    const int tok0 = t_begin + n * kSliceTok;
    const int page = bt[tok0 >> 6];
    const char* src = cache + static_cast<int64_t>(page) * (kPage * kRowBytes) +
                      (tok0 & (kPage - 1)) * kRowBytes;
    const uint32_t dst = lds_base + (n % kStages) * kSlotBytes + kLoadsPerWave * w * 1024;
    const int nv = t_end - tok0;
    if (nv >= kSliceTok) {
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) dma16(src, dma_off(i), dst + i * 1024);
    } else {
      // tail slice: rows of tokens >= nv are filled from token 0 of the slice
      // (finite data, weight 0), so empty cache slots are never read.
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) {
        const int t = dma_token(i);
        const uint32_t off = dma_off(i);
        dma16(src, t < nv ? off : off - t * kRowBytes, dst + i * 1024);
      }
    }
  };

  // --- per-lane LDS read offsets (within a slot)
  const int sw = swz(q);  // rows q and q + 16 share it
  // QK^T A operand: token tb*16 + q, logical chunk 4ks + g
  const uint32_t qk_off0 = q * kRowBytes + 16 * ((g) ^ sw);       // even ks
  const uint32_t qk_off1 = q * kRowBytes + 16 * ((4 + g) ^ sw);   // odd ks
  // PV A operand (transposed read): token 4g + q/4 (+16), column 16cb + 4(q%4)
  const int vrow = 4 * g + (q >> 2);
  const int vsw = swz(vrow);
  const uint32_t pv_base = vrow * kRowBytes + 8 * (q & 1);
  const int pv_hc = (q & 3) >> 1;

  __shared__ int restart_flag;
  if (threadIdx.x == 0) restart_flag = 0;

  float4_t oacc[32][2];
  float m_ref[2], l_run[2];
  const float c2 = scale * kLog2e;

  // S^T[32 tokens x 32 heads] of one slot = Rows . Q^T.  36 steps (ks, tb); LDS
  // reads run kAhead steps ahead of their MFMAs; scheduling fences keep the
  // compiler from hoisting more of them.
  auto scores = [&](const char* slot, float4_t (&sacc)[2][2]) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) sacc[tb][hb] = float4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int kSteps = 36, kAhead = 4;
    auto off_of = [&](int st) -> uint32_t {
      const int ks = st >> 1, tb = st & 1;
      return tb * 16 * kRowBytes + 128 * (ks >> 1) + ((ks & 1) ? qk_off1 : qk_off0);
    };
    bf16x8 fa[kAhead];
#pragma unroll
    for (int st = 0; st < kAhead; ++st) fa[st] = lds_read128(slot, off_of(st));
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int ks = st >> 1, tb = st & 1;
      const bf16x8 a = fa[st % kAhead];
      if (st + kAhead < kSteps) fa[st % kAhead] = lds_read128(slot, off_of(st + kAhead));
      sacc[tb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][ks], sacc[tb][0], 0, 0, 0);
      sacc[tb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][ks], sacc[tb][1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Scaled scores (log2 units, masked) and their per-head maximum over the slice.
  auto scaled_max = [&](const float4_t (&sacc)[2][2], int nv, float (&x)[2][2][4], float (&mx)[2]) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float m = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tb * 16 + 4 * g + i;
          const float v = t < nv ? sacc[tb][hb][i] * c2 : -INFINITY;
          x[tb][hb][i] = v;
          m = fmaxf(m, v);
        }
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      mx[hb] = m;
    }
  };

  // One pass over the item's slices through the LDS ring.
  //  kFull = true:  scores, weights p = 2^(x - m_ref), O += C^T P^T.  With
  //                 `first` the reference m_ref is the first slice's maximum and
  //                 a jump beyond max_jump aborts the pass (returns false).
  //  kFull = false: scores only, m_ref = exact per-head maximum.
  auto run_pass = [&](auto full_tag, bool first) -> bool {
    constexpr bool kFull = decltype(full_tag)::value;
    for (int n = 0; n < kStages - 1 && n < n_slices; ++n) issue(n);
    bool aborted = false;
    for (int n = 0; n < n_slices; ++n) {
      const int ahead = min(kStages - 2, n_slices - 1 - n);
      if (ahead >= 2)
        __builtin_amdgcn_s_waitcnt(MLA_VMCNT(2 * kLoadsPerWave));
      else if (ahead == 1)
        __builtin_amdgcn_s_waitcnt(MLA_VMCNT(kLoadsPerWave));
      else
        __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
      __syncthreads();
      if (kFull && first && restart_flag) {  // same value in every wave after the barrier
        aborted = true;
        break;
      }
      if (n + kStages - 1 < n_slices) issue(n + kStages - 1);

      const char* slot = lds + (n % kStages) * kSlotBytes;
      const int nv = min(kSliceTok, t_end - (t_begin + n * kSliceTok));
      float4_t sacc[2][2];
      scores(slot, sacc);
      float x[2][2][4], mx[2];
      scaled_max(sacc, nv, x, mx);
      if (!kFull) {
        m_ref[0] = fmaxf(m_ref[0], mx[0]);
        m_ref[1] = fmaxf(m_ref[1], mx[1]);
        continue;
      }
      if (first) {
        if (n == 0) {
          m_ref[0] = mx[0];
          m_ref[1] = mx[1];
        }
        if (__any(mx[0] > m_ref[0] + max_jump || mx[1] > m_ref[1] + max_jump)) {
          if (lane == 0) restart_flag = 1;
          continue;  // this pass will be discarded
        }
      }
      bf16x8 pf[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        uint32_t pk[4];
        float sum = 0.f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = bf16_bits_to_f32(f32_to_bf16_bits(exp2f(x[tb][hb][i] - m_ref[hb])));
            sum += p[i];
          }
          pk[2 * tb] = pack_bf16x2(p[0], p[1]);
          pk[2 * tb + 1] = pack_bf16x2(p[2], p[3]);
        }
        l_run[hb] += sum;
        pf[hb] = __builtin_bit_cast(bf16x8, pk);
      }
      // O^T[512 x 32 heads] += C^T . P^T, 32 steps of 16 latent columns
      constexpr int kSteps = 32, kAhead = 3;
      bf16x4 f0[kAhead], f1[kAhead];
      auto pv_off = [&](int cb) -> uint32_t {
        return pv_base + 128 * (cb >> 2) + 16 * ((2 * (cb & 3) + pv_hc) ^ vsw);
      };
#pragma unroll
      for (int cb = 0; cb < kAhead; ++cb) {
        f0[cb] = lds_read_tr(slot, pv_off(cb));
        f1[cb] = lds_read_tr(slot, pv_off(cb) + 16 * kRowBytes);
      }
#pragma unroll
      for (int cb = 0; cb < kSteps; ++cb) {
        const bf16x8 a = __builtin_shufflevector(f0[cb % kAhead], f1[cb % kAhead], 0, 1, 2, 3, 4, 5, 6, 7);
        if (cb + kAhead < kSteps) {
          f0[cb % kAhead] = lds_read_tr(slot, pv_off(cb + kAhead));
          f1[cb % kAhead] = lds_read_tr(slot, pv_off(cb + kAhead) + 16 * kRowBytes);
        }
        oacc[cb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[0], oacc[cb][0], 0, 0, 0);
        oacc[cb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[1], oacc[cb][1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (aborted) __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));  // loads of abandoned slices
    __syncthreads();  // ring free again; restart_flag final
    return !(kFull && first && restart_flag);
  };

  auto zero_state = [&]() {
#pragma unroll
    for (int cb = 0; cb < 32; ++cb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) oacc[cb][hb] = float4_t{0.f, 0.f, 0.f, 0.f};
    l_run[0] = l_run[1] = 0.f;
  };

  zero_state();
  if (!run_pass(std::integral_constant<bool, true>{}, true)) {
    // A head's maximum jumped by more than max_jump: take the exact maxima
    // first, then redo the item with them (every weight <= 1).
    m_ref[0] = m_ref[1] = -INFINITY;
    run_pass(std::integral_constant<bool, false>{}, false);
    zero_state();
    run_pass(std::integral_constant<bool, true>{}, false);
  }

  // ---- epilogue: normalise, write the partial
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    float l = l_run[hb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = 1.f / l;
    const int head = 32 * w + 16 * hb + q;
    float* orow = o_part + (static_cast<int64_t>(it) * H + head) * kDc + 4 * g;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      float4_t v = oacc[cb][hb];
      v[0] *= inv;
      v[1] *= inv;
      v[2] *= inv;
      v[3] *= inv;
      *reinterpret_cast<float4_t*>(orow + 16 * cb) = v;
    }
    if (g == 0) lse_part[static_cast<int64_t>(it) * H + head] = m_ref[hb] * kLn2 + logf(l);
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

hipError_t decode_fast(const mla_dims& d, const void* q_abs, const void* kv_cache,
                       const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                       const int32_t* items, int num_items, float* o_part, float* lse_part,
                       hipStream_t stream) {
  if (d.n_heads == 128) {
    hipLaunchKernelGGL(decode_h128_kernel, dim3(num_items), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q_abs), static_cast<const char*>(kv_cache),
                       block_table, max_pages, seq_lens, items, d.softmax_scale, max_jump(),
                       o_part, lse_part);
    return hipGetLastError();
  }
  return decode_generic(d, q_abs, kv_cache, block_table, max_pages, seq_lens, items, num_items,
                        o_part, lse_part, stream);
}

}  // namespace mla
