// Split-KV work planner (host only, integer arithmetic, deterministic).
//
// Every sequence's pages 0 .. ceil(L_b / page_size) - 1 are cut into contiguous,
// near-equal page ranges ("work items"); one workgroup decodes one item and
// writes one partial (o, lse) that the combine step merges.  More items fill
// more of the machine but each one adds a fixed cost (pipeline start-up and the
// partial's write + re-read), so the item size is picked by simulating the
// dispatch of the items onto `num_slots` workgroup slots and keeping the size
// with the shortest simulated makespan.  Items are dispatched in their own
// order (sequence by sequence), or, when the caller asks for a dispatch
// order, longest first, which the simulation then follows.
#include <algorithm>
#include <cstdint>
#include <functional>
#include <queue>
#include <vector>

#include "mla_internal.h"

namespace mla {
namespace {

// Cost unit: 1/16 of one page's streaming time.
constexpr int64_t kUnit = 16;

struct Layout {
  int64_t chunk;  // max pages per item
  int64_t items;
  int64_t makespan;
};

// Number of items a sequence of `pages` pages is cut into at chunk size `chunk`.
inline int64_t parts_of(int64_t pages, int64_t chunk) { return (pages + chunk - 1) / chunk; }

// Pages of part `k` when `pages` are cut into `n` near-equal parts (the first
// pages % n parts get one page more).
inline int64_t part_pages(int64_t pages, int64_t n, int64_t k) {
  return pages / n + (k < pages % n ? 1 : 0);
}

// Stops as soon as the makespan passes `bound` (a size already known to be
// worse needs no finishing).
Layout simulate(const std::vector<int64_t>& pages, int64_t chunk, int num_slots,
                int64_t overhead, int64_t bound) {
  Layout r{chunk, 0, 0};
  std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
  for (int i = 0; i < num_slots; ++i) free_at.push(0);
  for (int64_t p : pages) {
    const int64_t n = parts_of(p, chunk);
    for (int64_t k = 0; k < n; ++k) {
      const int64_t t = free_at.top();
      free_at.pop();
      const int64_t end = t + part_pages(p, n, k) * kUnit + overhead;
      r.makespan = std::max(r.makespan, end);
      if (r.makespan > bound) return r;
      free_at.push(end);
      ++r.items;
    }
  }
  return r;
}

// Longest-first dispatch (the items sorted by decreasing size) onto
// `num_slots` slots as the hardware places them: slot s of the dispatch order
// runs on XCD s % kXcds, and each XCD starts its items in order on its
// num_slots / kXcds slots as they free up.
constexpr int kXcds = 8;

// Item sizes (pages) of every sequence cut at `chunk`, longest first; ties keep
// the item order (sequence, then token order).
std::vector<int64_t> lpt_sizes(const std::vector<int64_t>& pages, int64_t chunk) {
  std::vector<int64_t> sz;
  for (int64_t p : pages) {
    const int64_t n = parts_of(p, chunk);
    for (int64_t k = 0; k < n; ++k) sz.push_back(part_pages(p, n, k));
  }
  std::stable_sort(sz.begin(), sz.end(), std::greater<int64_t>());
  return sz;
}

Layout simulate_lpt(const std::vector<int64_t>& pages, int64_t chunk, int num_slots,
                    int64_t overhead, int64_t bound) {
  Layout r{chunk, 0, 0};
  const std::vector<int64_t> sz = lpt_sizes(pages, chunk);
  const int per_xcd = std::max(1, num_slots / kXcds);
  std::vector<std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>>> free_at(kXcds);
  for (auto& q : free_at)
    for (int i = 0; i < per_xcd; ++i) q.push(0);
  for (size_t s = 0; s < sz.size(); ++s) {
    auto& q = free_at[s % kXcds];
    const int64_t t = q.top();
    q.pop();
    const int64_t end = t + sz[s] * kUnit + overhead;
    r.makespan = std::max(r.makespan, end);
    if (r.makespan > bound) return r;
    q.push(end);
    ++r.items;
  }
  return r;
}

}  // namespace

int64_t plan_max_items(int page_size, int batch, const int32_t* seq_lens) {
  if (page_size < 1 || batch < 1 || !seq_lens) return -1;
  int64_t n = 0;
  for (int b = 0; b < batch; ++b) {
    if (seq_lens[b] < 1) return -1;
    n += (static_cast<int64_t>(seq_lens[b]) + page_size - 1) / page_size;
  }
  return n;
}

mla_status plan_splits(int page_size, int batch, const int32_t* seq_lens, int num_slots,
                       int max_items, int32_t* items, int32_t* split_offsets, int32_t* num_items,
                       int n_heads, int32_t* order) {
  if (!seq_lens || !items || !split_offsets || !num_items) return MLA_ERR_INVALID_ARG;
  if (page_size < 1 || batch < 1 || num_slots < 1 || max_items < 0 || n_heads < 1)
    return MLA_ERR_INVALID_ARG;
  std::vector<int64_t> pages(batch);
  int64_t total = 0, longest = 0;
  for (int b = 0; b < batch; ++b) {
    if (seq_lens[b] < 1) return MLA_ERR_INVALID_ARG;
    pages[b] = (static_cast<int64_t>(seq_lens[b]) + page_size - 1) / page_size;
    total += pages[b];
    longest = std::max(longest, pages[b]);
  }
  if (total > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  // Fixed per-item cost: about one page of pipeline start-up plus the partial
  // (n_heads x (d_latent + 1) float32 written and read back) measured in pages
  // of 64 rows x 1152 bytes.
  const int64_t partial_bytes = static_cast<int64_t>(n_heads) * 513 * 4 * 2;
  const int64_t overhead = kUnit + (partial_bytes * kUnit) / (64 * 1152);

  // Candidate item sizes: about total / (k * num_slots) pages for k from 1 to 8
  // in steps of 1/16 (k waves of items), plus the longest sequence (no split).
  // The makespan changes by several percent between neighbouring sizes when
  // lengths are mixed, so the grid is fine.  Equal sizes are tried once, the
  // larger ones (fewer items, quicker to simulate) first, so that a good
  // makespan early cuts the simulation of worse sizes short.
  Layout best{longest, 0, INT64_MAX};
  std::vector<int64_t> cands;
  for (int j = 16; j <= 128; ++j) {
    const int64_t den = int64_t(j) * num_slots;
    // sizes past the longest sequence all give one item per sequence
    cands.push_back(std::min(longest, std::max<int64_t>(1, (total * 16 + den - 1) / den)));
  }
  cands.push_back(longest);
  std::sort(cands.begin(), cands.end(), std::greater<int64_t>());
  cands.erase(std::unique(cands.begin(), cands.end()), cands.end());
  for (int64_t c : cands) {
    Layout l = order ? simulate_lpt(pages, c, num_slots, overhead, best.makespan)
                     : simulate(pages, c, num_slots, overhead, best.makespan);
    if (l.makespan < best.makespan || (l.makespan == best.makespan && l.items < best.items)) best = l;
  }
  if (best.items > max_items) {
    *num_items = static_cast<int32_t>(best.items);
    return MLA_ERR_WORKSPACE;
  }
  int32_t w = 0;
  for (int b = 0; b < batch; ++b) {
    split_offsets[b] = w;
    const int64_t n = parts_of(pages[b], best.chunk);
    int64_t p0 = 0;
    for (int64_t k = 0; k < n; ++k) {
      const int64_t np = part_pages(pages[b], n, k);
      items[4 * w + 0] = b;
      items[4 * w + 1] = static_cast<int32_t>(k);
      items[4 * w + 2] = static_cast<int32_t>(p0);
      items[4 * w + 3] = static_cast<int32_t>(p0 + np);
      p0 += np;
      ++w;
    }
  }
  split_offsets[batch] = w;
  *num_items = w;
  if (order) {
    // longest first; among equal sizes, item order
    for (int32_t i = 0; i < w; ++i) order[i] = i;
    std::stable_sort(order, order + w, [&](int32_t a, int32_t b) {
      return items[4 * a + 3] - items[4 * a + 2] > items[4 * b + 3] - items[4 * b + 2];
    });
  }
  return MLA_OK;
}

}  // namespace mla
