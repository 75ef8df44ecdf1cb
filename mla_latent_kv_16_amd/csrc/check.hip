// Debug check of the device data that the decode and prefill entry points take
// on trust: the sequence lengths and the block-table entries they address.
//
// Page "DeepSeek V2 技术解析" 2.1.1 (paged KV memory: a sequence's tokens sit in
// fixed-size pages that a per-sequence table names).  Token j of sequence b is
// row j % page_size of page block_table[b][j / page_size]; the attention reads
// pages 0 .. ceil(L_b / page_size) - 1 of the row, so those entries must lie in
// [0, num_pages), and L_b in [min_len, max_pages_per_seq * page_size].
//
// One workgroup walks the [batch x max_pages_per_seq] table in a flat,
// coalesced loop; counts go through LDS atomics and thread 0 writes the two
// results, so the caller never has to clear the output first.
#include <limits.h>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void check_paging_kernel(
    int batch, int min_len, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ block_table, int max_pages, int page_size, int num_pages,
    int32_t* __restrict__ result) {
  __shared__ int s_bad;
  __shared__ int s_first;
  if (threadIdx.x == 0) {
    s_bad = 0;
    s_first = INT_MAX;
  }
  __syncthreads();
  const int64_t cap = static_cast<int64_t>(max_pages) * page_size;
  const int64_t n = static_cast<int64_t>(batch) * max_pages;
  int bad = 0, first = INT_MAX;
  for (int64_t e = threadIdx.x; e < n; e += kCheckThreads) {
    const int b = static_cast<int>(e / max_pages);
    const int p = static_cast<int>(e - static_cast<int64_t>(b) * max_pages);
    const int L = seq_lens[b];
    const bool len_ok = L >= min_len && L >= 1 && L <= cap;
    bool this_bad = false;
    if (!len_ok) {
      this_bad = (p == 0);  // one count per bad length; its entries mean nothing
    } else if (p < (static_cast<int64_t>(L) + page_size - 1) / page_size) {
      const int page = block_table[e];
      this_bad = page < 0 || page >= num_pages;
    }
    if (this_bad) {
      ++bad;
      first = min(first, b);
    }
  }
  if (bad) {
    atomicAdd(&s_bad, bad);
    atomicMin(&s_first, first);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    result[0] = s_bad;
    result[1] = s_bad ? s_first : -1;
  }
}

}  // namespace

hipError_t check_paging(const mla_dims& d, int batch, int min_len, const int32_t* seq_lens,
                        const int32_t* block_table, int max_pages, int num_pages,
                        int32_t* result, hipStream_t stream) {
  hipLaunchKernelGGL(check_paging_kernel, dim3(1), dim3(kCheckThreads), 0, stream, batch, min_len,
                     seq_lens, block_table, max_pages, d.page_size, num_pages, result);
  return hipGetLastError();
}

}  // namespace mla
