// Host driver for the split-KV planner, built with g++ under AddressSanitizer
// and UndefinedBehaviorSanitizer: every buffer it hands the planner is sized
// exactly (items: 4 x max_items, offsets: batch + 1), so any write past the
// capacity the planner was given, any read past the lengths array and any
// signed overflow or bad shift in its integer arithmetic aborts the run.
//
// It checks the plan's invariants itself: item b's pages cover
// 0 .. ceil(L_b / page_size) - 1 once, in order, in near-equal non-empty parts,
// and the CSR offsets are strictly increasing from 0 to the item count.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <vector>

#include "mla_internal.h"

namespace {

int g_failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                    \
    }                                                                  \
  } while (0)

// splitmix64: a fixed, portable generator for the random length mixes.
uint64_t next(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Plans `lens` twice: first with no room (the planner reports the count it
// needs), then with exactly that room; checks the result.
void plan_and_check(int page, const std::vector<int32_t>& lens, int slots, int heads,
                    bool ordered = false) {
  const int batch = static_cast<int>(lens.size());
  // the lengths live in an exactly sized heap block, so a read past batch is caught
  std::unique_ptr<int32_t[]> L(new int32_t[batch]);
  for (int b = 0; b < batch; ++b) L[b] = lens[b];
  std::unique_ptr<int32_t[]> offs(new int32_t[batch + 1]);
  std::unique_ptr<int32_t[]> none(new int32_t[0]);
  std::unique_ptr<int32_t[]> no_order(new int32_t[0]);
  int32_t need = -1;
  mla_status st = mla::plan_splits(page, batch, L.get(), slots, 0, none.get(), offs.get(), &need, heads,
                                   ordered ? no_order.get() : nullptr);
  EXPECT(st == MLA_ERR_WORKSPACE);
  EXPECT(need >= batch);
  const int64_t bound = mla::plan_max_items(page, batch, L.get());
  EXPECT(bound >= need);
  if (st != MLA_ERR_WORKSPACE || need < batch || bound < need) return;

  std::unique_ptr<int32_t[]> items(new int32_t[4 * static_cast<size_t>(need)]);
  std::unique_ptr<int32_t[]> order(new int32_t[static_cast<size_t>(need)]);
  int32_t got = -1;
  st = mla::plan_splits(page, batch, L.get(), slots, need, items.get(), offs.get(), &got, heads,
                        ordered ? order.get() : nullptr);
  EXPECT(st == MLA_OK);
  EXPECT(got == need);
  if (st != MLA_OK || got != need) return;

  EXPECT(offs[0] == 0);
  EXPECT(offs[batch] == got);
  for (int b = 0; b < batch; ++b) {
    const int32_t lo = offs[b], hi = offs[b + 1];
    EXPECT(hi > lo);
    if (hi <= lo) continue;
    const int64_t pages = (static_cast<int64_t>(L[b]) + page - 1) / page;
    int64_t p = 0, mn = INT64_MAX, mx = 0;
    for (int32_t i = lo; i < hi; ++i) {
      const int32_t* it = &items[4 * static_cast<size_t>(i)];
      EXPECT(it[0] == b);
      EXPECT(it[1] == i - lo);
      EXPECT(it[2] == p);
      EXPECT(it[3] > it[2]);
      const int64_t n = static_cast<int64_t>(it[3]) - it[2];
      mn = n < mn ? n : mn;
      mx = n > mx ? n : mx;
      p = it[3];
    }
    EXPECT(p == pages);
    EXPECT(mx - mn <= 1);
  }
  if (ordered) {
    // a permutation of the items, longest first, equal sizes in item order
    std::vector<char> seen(static_cast<size_t>(got), 0);
    for (int32_t s = 0; s < got; ++s) {
      const int32_t i = order[s];
      EXPECT(i >= 0 && i < got);
      if (i < 0 || i >= got) return;
      EXPECT(!seen[i]);
      seen[i] = 1;
      if (s > 0) {
        const int32_t j = order[s - 1];
        const int32_t si = items[4 * i + 3] - items[4 * i + 2], sj = items[4 * j + 3] - items[4 * j + 2];
        EXPECT(sj > si || (sj == si && j < i));
      }
    }
  }
}

void argument_errors() {
  int32_t L[2] = {100, 200}, offs[3], items[4 * 8], n = 0;
  EXPECT(mla::plan_splits(64, 2, nullptr, 256, 8, items, offs, &n, 128) == MLA_ERR_INVALID_ARG);
  EXPECT(mla::plan_splits(64, 2, L, 256, 8, nullptr, offs, &n, 128) == MLA_ERR_INVALID_ARG);
  EXPECT(mla::plan_splits(64, 2, L, 256, 8, items, nullptr, &n, 128) == MLA_ERR_INVALID_ARG);
  EXPECT(mla::plan_splits(64, 2, L, 256, 8, items, offs, nullptr, 128) == MLA_ERR_INVALID_ARG);
  EXPECT(mla::plan_splits(0, 2, L, 256, 8, items, offs, &n, 128) == MLA_ERR_INVALID_ARG);
  EXPECT(mla::plan_splits(64, 0, L, 256, 8, items, offs, &n, 128) == MLA_ERR_INVALID_ARG);
  EXPECT(mla::plan_splits(64, 2, L, 0, 8, items, offs, &n, 128) == MLA_ERR_INVALID_ARG);
  EXPECT(mla::plan_splits(64, 2, L, 256, -1, items, offs, &n, 128) == MLA_ERR_INVALID_ARG);
  EXPECT(mla::plan_splits(64, 2, L, 256, 8, items, offs, &n, 0) == MLA_ERR_INVALID_ARG);
  int32_t bad[2] = {100, 0};
  EXPECT(mla::plan_splits(64, 2, bad, 256, 8, items, offs, &n, 128) == MLA_ERR_INVALID_ARG);
  bad[1] = -5;
  EXPECT(mla::plan_splits(64, 2, bad, 256, 8, items, offs, &n, 128) == MLA_ERR_INVALID_ARG);
  EXPECT(mla::plan_max_items(64, 2, bad) == -1);
  EXPECT(mla::plan_max_items(0, 2, L) == -1);
  EXPECT(mla::plan_max_items(64, 0, L) == -1);
  EXPECT(mla::plan_max_items(64, 2, nullptr) == -1);
  // more pages than an int32 item field can index: refused before any planning
  int32_t huge[2] = {INT32_MAX, INT32_MAX};
  EXPECT(mla::plan_splits(1, 2, huge, 256, 8, items, offs, &n, 128) == MLA_ERR_UNSUPPORTED);
  // the largest lengths at the largest page size: no overflow in the rounding
  EXPECT(mla::plan_max_items(INT32_MAX, 2, huge) == 2);
}

}  // namespace

int main() {
  argument_errors();
  // edge lengths: one token, one page, one page and a token, long, mixed
  const std::vector<std::vector<int32_t>> fixed = {
      {1}, {64}, {65}, {32768}, {1, 64, 65, 32768}, std::vector<int32_t>(32, 4096),
      std::vector<int32_t>(64, 8192), std::vector<int32_t>(8, 131072), {INT32_MAX / 4}};
  for (const auto& lens : fixed)
    for (int heads : {16, 128})
      for (int slots : {1, 3, 256, 1024})
        for (bool ordered : {false, true}) plan_and_check(64, lens, slots, heads, ordered);
  // random mixes: batch 1..300, lengths 1..70000, page sizes 1..256
  uint64_t s = 20240611;
  for (int t = 0; t < 300; ++t) {
    const int batch = 1 + static_cast<int>(next(s) % 300);
    const int page = 1 + static_cast<int>(next(s) % 256);
    std::vector<int32_t> lens(batch);
    for (auto& l : lens) l = 1 + static_cast<int32_t>(next(s) % 70000);
    const int slots = 1 + static_cast<int>(next(s) % 2048);
    plan_and_check(page, lens, slots, (t & 1) ? 128 : 16, (t & 2) != 0);
  }
  if (g_failures) {
    std::printf("%d failures\n", g_failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
