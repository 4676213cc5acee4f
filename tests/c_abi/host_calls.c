/* A plain C caller of libcpattn's host-only entry points (no GPU, no
 * Python): the zigzag and interleave plans of the "Prefill Context
 * Parallelism" page's 16-token CP=4 examples, the restore index as the
 * inverse of the rank-major gathered order, the pass-KV / pass-Q threshold
 * of "What is Context Parallelism" section 3.5, ring padding, a workspace
 * query and the error paths.  Prints one line per check and "c abi OK";
 * exits non-zero on the first failure. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "cp_attn.h"

static int fails = 0;
#define CHECK(cond, what)                                  \
  do {                                                     \
    if (cond) {                                            \
      printf("ok   %s\n", what);                           \
    } else {                                               \
      printf("FAIL %s\n", what);                           \
      fails++;                                             \
    }                                                      \
  } while (0)

static int same(const int32_t *a, const int32_t *b, int n) {
  for (int i = 0; i < n; ++i)
    if (a[i] != b[i]) return 0;
  return 1;
}

int main(void) {
  cp_segment segs[8];
  int32_t pos[64], gidx[64], nseg = 0, nloc = 0, pad = 0;

  /* zigzag, CP=4, one request of 16 tokens: rank 0 owns {0,1,14,15} */
  const int32_t len16[1] = {16}, pre0[1] = {0};
  const int32_t want_z0[4] = {0, 1, 14, 15}, want_z2[4] = {4, 5, 10, 11};
  cp_status st = cp_shard_plan(CP_ZIGZAG, 4, 0, 1, len16, pre0, segs, 8, &nseg, pos, gidx, 64,
                               &nloc, &pad);
  CHECK(st == CP_OK && nloc == 4 && same(gidx, want_z0, 4) && nseg == 2, "zigzag rank 0");
  st = cp_shard_plan(CP_ZIGZAG, 4, 2, 1, len16, pre0, segs, 8, &nseg, pos, gidx, 64, &nloc, &pad);
  CHECK(st == CP_OK && nloc == 4 && same(gidx, want_z2, 4) && same(pos, want_z2, 4),
        "zigzag rank 2");

  /* interleave, CP=4, lengths 5 and 3 (no reset): rank 1 owns {1, 5} */
  const int32_t len53[2] = {5, 3}, pre00[2] = {0, 0};
  const int32_t want_i1[2] = {1, 5};
  st = cp_shard_plan(CP_INTERLEAVE, 4, 1, 2, len53, pre00, segs, 8, &nseg, pos, gidx, 64, &nloc,
                     &pad);
  CHECK(st == CP_OK && nloc == 2 && same(gidx, want_i1, 2), "interleave rank 1");
  /* index 5 is request 2's first token: position 0 */
  CHECK(pos[1] == 0, "interleave position restarts per request");

  /* restore: gathered (rank-major, padded) then gathered[restore[i]] == i */
  int32_t restore[16], gathered[64];
  st = cp_restore_index(CP_ZIGZAG, 4, 1, len16, restore, 16, &pad);
  CHECK(st == CP_OK && pad == 4, "restore index");
  for (int i = 0; i < 64; ++i) gathered[i] = -1;
  for (int r = 0; r < 4; ++r) {
    cp_shard_plan(CP_ZIGZAG, 4, r, 1, len16, pre0, segs, 8, &nseg, pos, gidx, 64, &nloc, &pad);
    for (int i = 0; i < nloc; ++i) gathered[r * pad + i] = gidx[i];
  }
  int ok = 1;
  for (int i = 0; i < 16; ++i) ok = ok && gathered[restore[i]] == i;
  CHECK(ok, "restore gathers the causal order");

  /* pass-KV / pass-Q: threshold 2 * 8 / 128 = 12.5 % */
  int32_t pass = -1;
  double miss = 0.0, h = 0.0;
  st = cp_choose_pass(16384, 114688, 128, 8, &pass, &miss, &h);
  CHECK(st == CP_OK && pass == CP_PASS_Q && miss == 0.125, "pass-Q at a 12.5 % miss rate");
  st = cp_choose_pass(16385, 114687, 128, 8, &pass, NULL, NULL);
  CHECK(st == CP_OK && pass == CP_PASS_KV, "pass-KV just above it");
  CHECK(cp_choose_pass(0, 1, 128, 8, &pass, NULL, NULL) == CP_ERR_ARG, "choose_pass rejects T = 0");

  /* ring padding: max P_i + ceil(T / N) */
  const int64_t cached[3] = {100, 300, 200};
  int64_t pad_len = 0;
  st = cp_ring_pad_len(3, cached, 10, &pad_len);
  CHECK(st == CP_OK && pad_len == 304, "ring pad length");

  /* workspace query of a bf16 call (host only): one int32 flag per workgroup */
  cp_segment one = {0, 0, 4, 0, 1, 0, 4};
  cp_attn_args a;
  memset(&a, 0, sizeof a);
  a.dtype = CP_BF16; a.o_dtype = CP_BF16; a.num_q_rows = 4; a.num_kv_rows = 4;
  a.hq = 4; a.hkv = 2; a.dqk = 128; a.dv = 128; a.scale = 0.1f; a.causal = 1;
  a.q_row_stride = 512; a.q_head_stride = 128; a.k_row_stride = 256; a.k_head_stride = 128;
  a.v_row_stride = 256; a.v_head_stride = 128; a.o_row_stride = 512; a.o_head_stride = 128;
  a.lse_row_stride = 4; a.segs = &one; a.num_segs = 1;
  size_t bytes = 0;
  st = cp_attn_workspace_size(&a, &bytes);
  CHECK(st == CP_OK && bytes == 16, "workspace query");
  a.hq = 3;
  CHECK(cp_attn_workspace_size(&a, &bytes) == CP_ERR_ARG, "hq % hkv != 0 rejected");

  /* argument errors and names */
  CHECK(cp_shard_plan(CP_ZIGZAG, 4, 4, 1, len16, pre0, segs, 8, &nseg, pos, gidx, 64, &nloc,
                      &pad) == CP_ERR_ARG, "rank out of range rejected");
  CHECK(cp_shard_plan(7, 4, 0, 1, len16, pre0, segs, 8, &nseg, pos, gidx, 64, &nloc, &pad) ==
            CP_ERR_ARG, "unknown strategy rejected");
  CHECK(cp_shard_plan(CP_ZIGZAG, 4, 0, 1, len16, pre0, segs, 1, &nseg, pos, gidx, 64, &nloc,
                      &pad) == CP_ERR_SMALL_BUFFER && nseg == 2,
        "small segment capacity reports the size");
  CHECK(strncmp(cp_status_str(CP_ERR_ARG), "CP_ERR_ARG", 10) == 0, "status names");
  CHECK(cp_version() != NULL && strlen(cp_version()) > 0, "version");

  if (fails) {
    printf("c abi: %d failures\n", fails);
    return 1;
  }
  printf("c abi OK\n");
  return 0;
}
