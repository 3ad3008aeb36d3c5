/* Every host-side check of the C ABI, driven from C: geometry validation,
 * workspace sizing and the refusal of each entry point's bad arguments.  No
 * call here passes validation, so nothing is launched and no GPU is needed;
 * the pointers are aligned addresses that are never dereferenced.  Built
 * against an AddressSanitizer / UndefinedBehaviorSanitizer build of the
 * library's host code, it checks that code for memory and UB errors.
 * Exit status: 0, or the number of the failed check. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdn.h"

static gdn_geometry base(void) {
  gdn_geometry g;
  memset(&g, 0, sizeof g);
  g.n_k_heads = 16;
  g.n_v_heads = 48;
  g.d_k = 128;
  g.d_v = 128;
  g.conv_width = 4;
  g.conv_channels = 2 * 16 * 128 + 48 * 128;
  g.conv_ring = 8;
  g.max_draft = 4;
  g.n_slots = 8;
  g.dtype_in = GDN_BF16;
  g.dtype_out = GDN_BF16;
  g.flags = GDN_FLAG_L2NORM_QK;
  g.q_scale = 1.0f;
  g.l2_eps = 1e-6f;
  return g;
}

#define P ((void*)(uintptr_t)0x10000)
#define PF ((float*)(uintptr_t)0x10000)
#define PI ((int32_t*)(uintptr_t)0x10000)
#define CHECK(id, cond)                                                     \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "check %d failed: %s (%s)\n", id, #cond, gdn_last_error()); \
      return id;                                                            \
    }                                                                       \
  } while (0)

static int has(const char* needle) { return strstr(gdn_last_error(), needle) != NULL; }

int main(void) {
  char msg[256];
  gdn_geometry g = base();
  CHECK(1, gdn_check_geometry(&g, msg, sizeof msg) == GDN_OK);
  CHECK(2, gdn_check_geometry(NULL, msg, sizeof msg) == GDN_ERR_NULL);
  /* every geometry field out of range, with a short message buffer too */
  struct { int field; int value; gdn_status st; } cases[] = {
      {0, 47, GDN_ERR_GEOMETRY}, {1, 10000, GDN_ERR_GEOMETRY}, {2, 6, GDN_ERR_GEOMETRY},
      {2, 4, GDN_ERR_GEOMETRY},  {3, 5, GDN_ERR_GEOMETRY},     {4, 0, GDN_ERR_GEOMETRY},
      {5, 0, GDN_ERR_GEOMETRY},  {6, 7, GDN_ERR_GEOMETRY},     {7, 6, GDN_ERR_GEOMETRY},
      {8, 96, GDN_ERR_UNSUPPORTED}, {9, 0, GDN_ERR_GEOMETRY},  {10, -3, GDN_ERR_GEOMETRY}};
  for (unsigned i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
    gdn_geometry b = base();
    switch (cases[i].field) {
      case 0: b.n_v_heads = cases[i].value; break;
      case 1: b.conv_channels = cases[i].value; break;
      case 2: b.conv_ring = cases[i].value; break;
      case 3: b.conv_width = cases[i].value; break;
      case 4: b.max_draft = cases[i].value; break;
      case 5: b.n_slots = cases[i].value; break;
      case 6: b.dtype_in = cases[i].value; break;
      case 7: b.flags = (uint32_t)cases[i].value; break;
      case 8: b.d_k = b.d_v = cases[i].value; b.conv_channels = 2 * 16 * 96 + 48 * 96; break;
      case 9: b.n_k_heads = cases[i].value; break;
      case 10: b.d_k = cases[i].value; break;
    }
    CHECK(100 + (int)i, gdn_check_geometry(&b, msg, sizeof msg) == cases[i].st);
    CHECK(200 + (int)i, gdn_check_geometry(&b, msg, 8) == cases[i].st && strlen(msg) <= 7);
    CHECK(300 + (int)i, gdn_check_geometry(&b, NULL, 0) == cases[i].st);
  }
  /* workspace sizes: bounded in n_tokens, zero for a bad geometry */
  size_t w1 = gdn_prefill_workspace_bytes(&g, 8192, 1), w2 = gdn_prefill_workspace_bytes(&g, 1 << 20, 8);
  CHECK(3, w1 > 0 && w1 == w2);
  CHECK(4, gdn_prefill_workspace_bytes(NULL, 8192, 1) == 0);
  g.n_v_heads = 47;
  CHECK(5, gdn_prefill_workspace_bytes(&g, 8192, 1) == 0);
  g = base();

  /* decode */
  CHECK(10, gdn_decode_step(&g, PF, PF, PI, P, P, P, PF, PI, 0, P, NULL, NULL) == GDN_ERR_RANGE && has("batch: 0"));
  CHECK(11, gdn_decode_step(&g, PF, PF, PI, P, P, P, PF, PI, 9, P, NULL, NULL) == GDN_ERR_RANGE);
  CHECK(12, gdn_decode_step(&g, NULL, PF, PI, P, P, P, PF, PI, 4, P, NULL, NULL) == GDN_ERR_NULL && has("state"));
  CHECK(13, gdn_decode_step(&g, PF, PF, PI, (char*)P + 2, P, P, PF, PI, 4, P, NULL, NULL) == GDN_ERR_ALIGN);
  CHECK(14, gdn_decode_step(&g, PF, PF, PI, P, P, P, NULL, PI, 4, P, NULL, NULL) == GDN_ERR_NULL);
  CHECK(15, gdn_decode_step(NULL, PF, PF, PI, P, P, P, PF, PI, 4, P, NULL, NULL) == GDN_ERR_NULL);
  /* conv-state step */
  CHECK(20, gdn_conv_state_step(&g, PF, PI, P, PF, PI, 0, P, NULL, NULL) == GDN_ERR_RANGE);
  CHECK(21, gdn_conv_state_step(&g, NULL, PI, P, PF, PI, 4, P, NULL, NULL) == GDN_ERR_NULL);
  /* verify and rollback */
  CHECK(30, gdn_verify_k(&g, PF, PF, PI, P, P, P, PF, PI, 4, 0, PF, P, NULL, NULL) == GDN_ERR_RANGE);
  CHECK(31, gdn_verify_k(&g, PF, PF, PI, P, P, P, PF, PI, 4, 5, PF, P, NULL, NULL) == GDN_ERR_RANGE &&
                has("k: 5, required: 1..max_draft = 4"));
  CHECK(32, gdn_verify_k(&g, PF, PF, PI, P, P, P, PF, PI, 4, 4, NULL, P, NULL, NULL) == GDN_ERR_NULL);
  CHECK(33, gdn_rollback(&g, PF, PI, PF, PI, NULL, 4, 4, NULL, NULL) == GDN_ERR_NULL && has("accepted"));
  CHECK(34, gdn_rollback(&g, PF, PI, PF, PI, PI, 0, 4, NULL, NULL) == GDN_ERR_RANGE);
  CHECK(35, gdn_verify_k_slots(&g, PF, PF, PI, P, P, P, PF, PI, 4, 0, PI, PI, P, NULL, NULL) == GDN_ERR_RANGE);
  CHECK(36, gdn_commit_slots(&g, PI, PI, NULL, PI, 4, 4, PI, NULL, NULL) == GDN_ERR_NULL);
  /* prefill, with and without checkpoints, and without a workspace */
  CHECK(40, gdn_prefill_chunked(&g, PF, PF, PI, P, P, P, PF, PI, PI, PI, 1, 8192, 128, P, w1, P, NULL, NULL) ==
                GDN_ERR_UNSUPPORTED && has("chunk: 128"));
  CHECK(41, gdn_prefill_chunked(&g, PF, PF, PI, P, P, P, PF, PI, PI, PI, 1, 8192, 64, P, w1 - 1, P, NULL, NULL) ==
                GDN_ERR_WORKSPACE);
  CHECK(42, gdn_prefill_chunked(&g, PF, PF, PI, P, P, P, PF, PI, PI, PI, 9, 8192, 64, P, w1, P, NULL, NULL) ==
                GDN_ERR_RANGE);
  CHECK(43, gdn_prefill_chunked(&g, PF, PF, PI, P, P, P, PF, PI, PI, PI, 1, -1, 64, P, w1, P, NULL, NULL) ==
                GDN_ERR_RANGE);
  CHECK(44, gdn_prefill_chunked(&g, PF, PF, PI, P, P, P, PF, NULL, PI, PI, 1, 8192, 64, P, w1, P, NULL, NULL) ==
                GDN_ERR_NULL);
  CHECK(45, gdn_prefill_chunked_ckpt(&g, PF, PF, PI, P, P, P, PF, PI, PI, PI, 1, 8192, 64, P, w1, P, 0, PF,
                                     (size_t)1 << 30, NULL, NULL) == GDN_ERR_RANGE && has("ckpt_every: 0"));
  CHECK(46, gdn_prefill_chunked_ckpt(&g, PF, PF, PI, P, P, P, PF, PI, PI, PI, 1, 8192, 64, P, w1, P, 512, PF, 16,
                                     NULL, NULL) == GDN_ERR_RANGE && has("ckpt_bytes"));
  gdn_geometry big = base();
  big.n_k_heads = 64;
  big.n_v_heads = 192;
  big.conv_channels = 2 * 64 * 128 + 192 * 128;
  CHECK(47, gdn_prefill_chunked_static(&big, PF, PF, PI, P, P, P, PF, PI, PI, PI, 1, 8192, 64, P, NULL, NULL) ==
                GDN_ERR_WORKSPACE && has("static workspace"));
  g.dtype_in = g.dtype_out = GDN_F32;
  CHECK(48, gdn_prefill_chunked(&g, PF, PF, PI, P, P, P, PF, PI, PI, PI, 1, 8192, 64, P, w1, P, NULL, NULL) ==
                GDN_ERR_UNSUPPORTED);
  /* kernel-timing requests: both events or neither; consumed by the next prefill call */
  CHECK(60, gdn_prefill_timing_events(P, NULL) == GDN_ERR_NULL && has("stop is null"));
  CHECK(61, gdn_prefill_timing_events(NULL, P) == GDN_ERR_NULL);
  CHECK(62, gdn_prefill_timing_events(P, P) == GDN_OK);
  CHECK(63, gdn_prefill_chunked(&g, PF, PF, PI, P, P, P, PF, PI, PI, PI, 1, 8192, 128, P, w1, P, NULL, NULL) ==
                GDN_ERR_UNSUPPORTED);
  CHECK(64, gdn_prefill_timing_events(NULL, NULL) == GDN_OK);
  /* strings */
  for (int s = -1; s <= 8; ++s) CHECK(50, gdn_status_string((gdn_status)s) != NULL);
  CHECK(51, strcmp(gdn_status_string(GDN_ERR_WORKSPACE), "GDN_ERR_WORKSPACE") == 0);
  printf("abi refusals ok\n");
  return 0;
}
