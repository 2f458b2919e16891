/*
 * c_abi_check.c -- the C ABI of include/cpattn.h used from plain C11, without a GPU.
 *
 * Built and run by tests/test_abi.py (gcc -std=c11 -pedantic -Werror, linked against
 * libcpattn.so). It exercises only host-side behaviour: the shard map, argument validation that
 * rejects a call before any launch, a call with nothing to do, the workspace size and the ring
 * variant selector. Prints "ok" and exits 0 when every check holds.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "cpattn.h"

static int failures = 0;

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

/* Load-balanced chunking of one 257-token sequence over 4 ranks: every token owned exactly once,
 * rank r holding chunk r then chunk 7 - r with floor edges. */
static void check_shard_map(void) {
  const int64_t begin = 0, end = 257;
  const int world = 4;
  int owner[257];
  for (int i = 0; i < 257; ++i) owner[i] = -1;
  for (int r = 0; r < world; ++r) {
    cp_segment segs[4];
    int n_segs = 0;
    int64_t toks[128];
    int64_t n_tok = 0;
    const int st = cp_shard_map(1, NULL, &begin, &end, world, r, segs, 4, &n_segs, toks, 128, &n_tok);
    CHECK(st == CP_OK);
    CHECK(n_segs == 2);
    const int64_t c0 = r, c1 = 2 * world - 1 - r;
    CHECK(segs[0].pos_start == c0 * 257 / 8 && segs[0].len == (c0 + 1) * 257 / 8 - c0 * 257 / 8);
    CHECK(segs[1].pos_start == c1 * 257 / 8 && segs[1].len == (c1 + 1) * 257 / 8 - c1 * 257 / 8);
    CHECK(segs[0].local_start == 0 && segs[1].local_start == segs[0].len);
    CHECK(n_tok == segs[0].len + segs[1].len);
    for (int64_t i = 0; i < n_tok; ++i) {
      CHECK(toks[i] >= 0 && toks[i] < 257);
      if (toks[i] >= 0 && toks[i] < 257) {
        CHECK(owner[toks[i]] == -1);
        owner[toks[i]] = r;
      }
    }
  }
  for (int i = 0; i < 257; ++i) CHECK(owner[i] != -1);

  /* too small a segment buffer: CP_E_CAPACITY with the required count reported */
  cp_segment one[1];
  int need = 0;
  CHECK(cp_shard_map(1, NULL, &begin, &end, world, 0, one, 1, &need, NULL, 0, NULL) == CP_E_CAPACITY);
  CHECK(need == 2);
  CHECK(strlen(cp_last_error()) > 0);
}

/* Validation happens before anything is launched, so these calls need no device. */
static void check_validation(void) {
  cp_segment seg;
  seg.seq_id = 0;
  seg.reserved = 0;
  seg.pos_start = 0;
  seg.len = 16;
  seg.local_start = 0;
  /* fake, 16-byte aligned addresses: never dereferenced, since every call below stops first */
  const void* q = (const void*)(uintptr_t)0x1000;
  float* o = (float*)(uintptr_t)0x2000;
  float* lse = (float*)(uintptr_t)0x3000;

  CHECK(cp_partial_attn(q, q, q, 16, 16, 6, 4, 64, CP_BF16, &seg, 1, &seg, 1, 1, 0.125f, o, lse, 0,
                        NULL) == CP_E_SHAPE);
  CHECK(strlen(cp_last_error()) > 0);
  CHECK(cp_partial_attn(q, q, q, 16, 16, 4, 1, 96, CP_BF16, &seg, 1, &seg, 1, 1, 0.125f, o, lse, 0,
                        NULL) == CP_E_UNSUPPORTED);
  CHECK(cp_partial_attn(q, q, q, 16, 16, 4, 1, 64, CP_BF16, &seg, 1, &seg, 1, 1, 0.0f, o, lse, 0,
                        NULL) == CP_E_ARG);
  seg.len = 17; /* runs past the 16-row shard */
  CHECK(cp_partial_attn(q, q, q, 16, 16, 4, 1, 64, CP_BF16, &seg, 1, &seg, 1, 1, 0.125f, o, lse, 0,
                        NULL) == CP_E_SHAPE);
  /* no query runs: nothing to do, nothing launched, success */
  CHECK(cp_partial_attn(q, q, q, 16, 16, 4, 1, 64, CP_BF16, &seg, 0, &seg, 0, 1, 0.125f, o, lse, 0,
                        NULL) == CP_OK);
  CHECK(strlen(cp_last_error()) == 0);

  const float* parts[1] = {o};
  CHECK(cp_merge_lse(0, parts, parts, 8, 64, o, CP_F32, NULL, NULL) == CP_E_CAPACITY);
  CHECK(cp_decode_splitkv(q, q, q, NULL, NULL, 2, 16, 1, 128, CP_F32, 256, 0.1f, o, lse, o, CP_F32,
                          NULL, NULL) == CP_E_UNSUPPORTED);
  CHECK(strcmp(cp_status_string(CP_E_SHAPE), "CP_E_SHAPE") == 0);
}

static void check_sizes_and_selector(void) {
  CHECK(cp_decode_workspace_bytes(32, 16, 128, 256) == (size_t)32 * 256 * 16 * (128 * 4 + 4));
  CHECK(cp_decode_workspace_bytes_ex(32, 16, 128, 256, CP_BF16) == (size_t)32 * 256 * 16 * (128 * 2 + 4));
  CHECK(cp_decode_workspace_bytes(-1, 16, 128, 256) == 0);

  int variant = -1, reason = -1;
  /* miss rate 100% > 2 * N_KV / N_H = 12.5%: Pass-KV by the first condition */
  CHECK(cp_select_ring_variant(1000, 0, 4, 16, 1, 128, 2, 153e9, 1.2e15, &variant, &reason) == CP_OK);
  CHECK(variant == CP_PASS_KV && reason == 1);
  CHECK(cp_select_ring_variant(0, 0, 4, 16, 1, 128, 2, 153e9, 1.2e15, &variant, &reason) == CP_E_ARG);
}

int main(void) {
  check_shard_map();
  check_validation();
  check_sizes_and_selector();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
