/* A C99 client of libmla that uses only host-side behaviour: the header must
 * compile as C, the library must link and load, the planner must cover every
 * page exactly once, and every device entry point must reject bad arguments
 * before touching the GPU (so this runs on a machine without one).
 * Prints "ok" and exits 0 on success; prints the first failure and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mla.h"

static int fails = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);          \
      fails++;                                                        \
    }                                                                 \
  } while (0)

int main(void) {
  mla_dims v2;
  memset(&v2, 0, sizeof v2);
  v2.n_heads = 128;
  v2.d_head = 128;
  v2.d_latent = 512;
  v2.d_rope = 64;
  v2.page_size = 64;
  v2.softmax_scale = 0.0721687836f; /* 1 / sqrt(192) */
  v2.rope_base = 10000.0;
  v2.dtype = MLA_BF16;

  CHECK(mla_version() > 0);
  CHECK(mla_status_string(MLA_OK) != NULL);
  CHECK(mla_status_string((mla_status)-99) != NULL);
  CHECK(mla_last_hip_error() != NULL);
  CHECK(mla_fast_path(&v2) == 1);
  {
    mla_dims odd = v2;
    odd.n_heads = 64; /* any multiple of 16 */
    CHECK(mla_fast_path(&odd) == 1);
    odd.n_heads = 40;
    CHECK(mla_fast_path(&odd) == 0);
    odd.d_rope = 63; /* must be even */
    CHECK(mla_fast_path(&odd) < 0);
  }

  /* planner: ragged lengths, every page exactly once, items in sequence order */
  {
    const int32_t lens[5] = {1, 64, 65, 8192, 30000};
    const int B = 5;
    int64_t cap = mla_plan_max_items(&v2, B, lens);
    int64_t pages_total = 0;
    for (int b = 0; b < B; ++b) pages_total += (lens[b] + 63) / 64;
    CHECK(cap == pages_total);
    int32_t* items = (int32_t*)calloc((size_t)cap * 4, sizeof(int32_t));
    int32_t offs[6];
    int32_t n = 0;
    CHECK(mla_plan_splits(&v2, B, lens, 256, (int32_t)cap, items, offs, &n) == MLA_OK);
    CHECK(n >= B && n <= cap);
    CHECK(offs[0] == 0 && offs[B] == n);
    for (int b = 0; b < B; ++b) {
      int32_t next = 0;
      for (int i = offs[b]; i < offs[b + 1]; ++i) {
        CHECK(items[4 * i] == b);
        CHECK(items[4 * i + 1] == i - offs[b]);
        CHECK(items[4 * i + 2] == next);
        CHECK(items[4 * i + 3] > items[4 * i + 2]);
        next = items[4 * i + 3];
      }
      CHECK(next == (lens[b] + 63) / 64);
    }
    /* too small a buffer: the capacity needed comes back, nothing else */
    int32_t small_items[4] = {0, 0, 0, 0};
    CHECK(mla_plan_splits(&v2, B, lens, 256, 1, small_items, offs, &n) == MLA_ERR_WORKSPACE);
    CHECK(n > 1);
    free(items);
  }

  /* device entry points: NULL pointers are rejected before any HIP call */
  {
    void* p = (void*)(uintptr_t)0x7f0000000000ull; /* aligned stand-in, never touched */
    float* f = (float*)p;
    const int32_t* i = (const int32_t*)p;
    CHECK(mla_absorb_q(&v2, 2, NULL, p, i, p, p, NULL) == MLA_ERR_INVALID_ARG);
    CHECK(mla_decode_splitkv(&v2, 2, NULL, p, 10, i, 4, i, i, 3, f, f, NULL) == MLA_ERR_INVALID_ARG);
    CHECK(mla_decode_splitkv_multi(&v2, 2, 0, p, p, 10, i, 4, i, i, 3, f, f, NULL) == MLA_ERR_INVALID_ARG);
    CHECK(mla_combine(&v2, 2, NULL, f, f, f, NULL, NULL) == MLA_ERR_INVALID_ARG);
    CHECK(mla_combine_multi(&v2, 2, 2, i, NULL, f, f, NULL, NULL) == MLA_ERR_INVALID_ARG);
    CHECK(mla_decode_merged(&v2, 2, p, p, 10, i, 4, i, i, 3, i, f, f, NULL, f, NULL, NULL) ==
          MLA_ERR_INVALID_ARG);
    CHECK(mla_out_proj(&v2, 2, f, NULL, f, NULL) == MLA_ERR_INVALID_ARG);
    CHECK(mla_combine_out_proj(&v2, 2, 1, i, f, f, p, NULL, NULL, NULL, NULL) == MLA_ERR_INVALID_ARG);
    CHECK(mla_append_kv(&v2, 5120, 2, p, p, p, i, 1, 1e-6f, p, 10, i, 4, NULL, 1 << 20, NULL) ==
          MLA_ERR_INVALID_ARG);
    CHECK(mla_append_kv_workspace_bytes(&v2, 5120, 64) == (int64_t)8 * 64 * 576 * 4);
    CHECK(mla_check_paging(&v2, 2, 1, i, 10, NULL, 4, (int32_t*)p, NULL) == MLA_ERR_INVALID_ARG);
  }

  if (fails) return 1;
  printf("ok\n");
  return 0;
}
