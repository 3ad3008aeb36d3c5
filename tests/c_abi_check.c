/* A plain C99 caller of the library's host-only entry points: the header is
 * valid C and the shared library links and answers without Python.  No GPU
 * work is launched (every call here is a host-side check). */
#include <stdio.h>
#include <string.h>

#include "gdn.h"

int main(void) {
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
  char msg[256];
  if (gdn_abi_version() != GDN_ABI_VERSION) return 10;
  if (gdn_check_geometry(&g, msg, sizeof msg) != GDN_OK) return 11;
  if (gdn_prefill_workspace_bytes(&g, 8192, 1) == 0) return 12;
  g.conv_channels += 1;
  if (gdn_check_geometry(&g, msg, sizeof msg) != GDN_ERR_GEOMETRY) return 13;
  if (strstr(msg, "conv_channels") == NULL) return 14;
  if (strcmp(gdn_status_string(GDN_ERR_GEOMETRY), "GDN_ERR_GEOMETRY") != 0) return 15;
  printf("c abi ok: %s\n", gdn_version());
  return 0;
}
