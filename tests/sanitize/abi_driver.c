/* Host driver for the sanitizer build of libmoe's argument checking: every entry point of moe.h
 * with invalid arguments, and with T = 0, so that AddressSanitizer and UndefinedBehaviorSanitizer
 * see the validation code of the C ABI. No call here reaches a GPU: each one fails validation or
 * has nothing to launch, and the pointers are host addresses that are never dereferenced.
 * Prints "abi driver ok" and exits 0 when every status is the documented one. */
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int fails = 0;

#define EXPECT(call, st)                                                                          \
  do {                                                                                            \
    moe_status s_ = (call);                                                                       \
    if (s_ != (st)) {                                                                             \
      fprintf(stderr, "FAILED %s: got %d, want %d (%s)\n", #call, (int)s_, (int)(st), moe_last_error()); \
      ++fails;                                                                                    \
    }                                                                                             \
  } while (0)

static _Alignas(256) char buf[1 << 12];

int main(void) {
  void* p = buf;          /* 256-byte aligned stand-in pointer, never dereferenced */
  void* mis = buf + 8;    /* misaligned */
  const moe_dims ok = {32, 4096, 14336, 8, 2, MOE_BF16, MOE_LAYOUT_ROWMAJOR};
  moe_dims d;

  /* dims */
  EXPECT(moe_route(NULL, NULL, p, p, p, p, NULL, NULL), MOE_ERR_INVALID_ARG);
  d = ok; d.K = 9;
  EXPECT(moe_route(&d, NULL, p, p, p, p, NULL, NULL), MOE_ERR_INVALID_ARG);
  d = ok; d.E = 65; d.K = 2;
  EXPECT(moe_route(&d, NULL, p, p, p, p, NULL, NULL), MOE_ERR_UNSUPPORTED);
  d = ok; d.d = 100;
  EXPECT(moe_route(&d, NULL, p, p, p, p, NULL, NULL), MOE_ERR_UNSUPPORTED);
  d = ok; d.T = -1;
  EXPECT(moe_route(&d, NULL, p, p, p, p, NULL, NULL), MOE_ERR_INVALID_ARG);
  d = ok; d.dtype = 7;
  EXPECT(moe_route(&d, NULL, p, p, p, p, NULL, NULL), MOE_ERR_INVALID_ARG);
  d = ok; d.weight_layout = 3;
  EXPECT(moe_expert_ffn(&d, p, p, p, p, p, p, p, NULL), MOE_ERR_INVALID_ARG);
  /* pointers */
  EXPECT(moe_route(&ok, NULL, mis, p, p, p, NULL, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_route(&ok, NULL, p, NULL, p, p, NULL, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_permute(&ok, p, p, p, p, p, NULL, NULL, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine(&ok, NULL, p, p, p, mis, NULL), MOE_ERR_INVALID_ARG);
  /* options */
  moe_opts bad = {NULL, 5, 0, NULL, NULL};
  EXPECT(moe_combine(&ok, &bad, p, p, p, p, NULL), MOE_ERR_INVALID_ARG);
  moe_opts acc = {NULL, MOE_BF16, 2, NULL, NULL};
  EXPECT(moe_forward(&ok, &acc, p, p, p, p, p, p, p, 1 << 30, NULL), MOE_ERR_INVALID_ARG);
  moe_opts act = {NULL, MOE_BF16, 0, NULL, (float*)mis};
  EXPECT(moe_forward(&ok, &act, p, p, p, p, p, p, p, 1 << 30, NULL), MOE_ERR_INVALID_ARG);
  /* workspace */
  const size_t need = moe_workspace_bytes(&ok);
  if (need == 0) { fprintf(stderr, "FAILED moe_workspace_bytes\n"); ++fails; }
  d = ok; d.K = 9;
  if (moe_workspace_bytes(&d) != 0) { fprintf(stderr, "FAILED moe_workspace_bytes(invalid)\n"); ++fails; }
  EXPECT(moe_forward(&ok, NULL, p, p, p, p, p, p, p, need - 1, NULL), MOE_ERR_WORKSPACE);
  EXPECT(moe_forward(&ok, NULL, p, p, p, p, p, p, mis, need, NULL), MOE_ERR_INVALID_ARG);
  d = ok; d.T = 4096;
  EXPECT(moe_forward_noalloc(&d, NULL, p, p, p, p, p, p, NULL), MOE_ERR_WORKSPACE);
  d = ok; d.K = 9;
  EXPECT(moe_forward_noalloc(&d, NULL, p, p, p, p, p, p, NULL), MOE_ERR_INVALID_ARG);
  /* packing */
  EXPECT(moe_pack_weights(&ok, 7, p, buf + 1024, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_pack_weights(&ok, MOE_W_UP, p, buf + 1024, NULL), MOE_ERR_INVALID_ARG); /* overlap */
  /* backward */
  d = ok; d.dtype = MOE_F32;
  EXPECT(moe_backward(&d, NULL, p, p, p, p, p, p, p, p, p, p, p, NULL, p, 1 << 30, NULL), MOE_ERR_UNSUPPORTED);
  d = ok; d.weight_layout = 2; /* not a layout */
  EXPECT(moe_backward(&d, NULL, p, p, p, p, p, p, p, p, p, p, p, NULL, p, 1 << 30, NULL), MOE_ERR_INVALID_ARG);
  d = ok; d.weight_layout = MOE_LAYOUT_PACKED; /* either layout: the same workspace */
  if (moe_backward_workspace_bytes(&d) != moe_backward_workspace_bytes(&ok)) {
    fprintf(stderr, "FAILED moe_backward_workspace_bytes (packed)\n");
    ++fails;
  }
  if (moe_backward_workspace_bytes(&ok) == 0) { fprintf(stderr, "FAILED moe_backward_workspace_bytes\n"); ++fails; }
  EXPECT(moe_backward(&ok, NULL, p, p, p, p, p, p, p, p, p, p, p, NULL, p, 16, NULL), MOE_ERR_WORKSPACE);
  /* norm, attention, block */
  EXPECT(moe_rmsnorm(4, 4096, -1.0f, (const float*)p, p, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_rmsnorm(4, 100, 1e-5f, (const float*)p, p, NULL), MOE_ERR_UNSUPPORTED);
  moe_attn_dims at = {32, 4096, 32, 8, 128, 1e6f, 1e-5f};
  moe_attn_dims at2 = at; at2.head_dim = 64;
  EXPECT(moe_attention(&at2, p, p, p, p, NULL), MOE_ERR_UNSUPPORTED);
  at2 = at; at2.n_kv_heads = 7;
  EXPECT(moe_attention(&at2, p, p, p, p, NULL), MOE_ERR_INVALID_ARG);
  at2 = at; at2.rope_base = 0.5f;
  EXPECT(moe_attention(&at2, p, p, p, p, NULL), MOE_ERR_INVALID_ARG);
  at2 = at; at2.T = 33;
  if (moe_block_workspace_bytes(&ok, &at2) != 0) { fprintf(stderr, "FAILED block workspace (T mismatch)\n"); ++fails; }
  EXPECT(moe_block_forward(&ok, &at2, NULL, (float*)p, p, p, p, p, p, p, p, 1 << 30, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_block_forward(&ok, &at, NULL, (float*)p, p, p, p, p, p, p, p, 16, NULL), MOE_ERR_WORKSPACE);
  /* T = 0: valid, nothing launched */
  d = ok; d.T = 0;
  EXPECT(moe_route(&d, NULL, p, p, p, p, NULL, NULL), MOE_OK);
  EXPECT(moe_permute(&d, p, p, p, p, p, p, NULL, NULL), MOE_OK);
  EXPECT(moe_expert_ffn(&d, p, p, p, p, p, p, p, NULL), MOE_OK);
  EXPECT(moe_combine(&d, NULL, p, p, p, p, NULL), MOE_OK);
  EXPECT(moe_forward(&d, NULL, p, p, p, p, p, p, NULL, 0, NULL), MOE_OK);
  EXPECT(moe_forward_noalloc(&d, NULL, p, p, p, p, p, p, NULL), MOE_OK);
  EXPECT(moe_backward(&d, NULL, p, p, p, p, p, p, p, p, p, p, p, NULL, NULL, 0, NULL), MOE_OK);
  EXPECT(moe_rmsnorm(0, 4096, 1e-5f, (const float*)p, p, NULL), MOE_OK);
  at2 = at; at2.T = 0;
  EXPECT(moe_attention(&at2, p, p, p, p, NULL), MOE_OK);
  /* strings */
  for (int s = 0; s <= 4; ++s)
    if (strncmp(moe_status_string((moe_status)s), "MOE_", 4) != 0) { fprintf(stderr, "FAILED status string\n"); ++fails; }
  if (strcmp(moe_status_string((moe_status)99), "MOE_STATUS_UNKNOWN") != 0) {
    fprintf(stderr, "FAILED unknown status string\n");
    ++fails;
  }
  if (moe_abi_version() != 5) { fprintf(stderr, "FAILED abi version\n"); ++fails; }
  if (fails) return 1;
  printf("abi driver ok\n");
  return 0;
}
