/* Host-side argument checks of libhstu under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built and run by tests/test_host_sanitizer.py,
 * CPU only).  Every call here must be refused, or sized, by the library's
 * host code before any device work: invalid descriptors and pointers,
 * extreme sizes (overflow in the size arithmetic would be reported by
 * UBSan), undersized workspaces.  Prints "ok" and exits 0 when every return
 * value is the documented one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "hstu.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static hstu_attn_desc desc(void) {
  hstu_attn_desc d;
  memset(&d, 0, sizeof d);
  d.B = 4; d.T = 300; d.H = 2; d.d_qk = 32; d.d_v = 32;
  d.n_pos_buckets = 128; d.n_time_buckets = 128; d.norm_mode = 0; d.norm_len = 128;
  d.dtype = HSTU_BF16; d.rab_head_stride = 128;
  return d;
}

int main(void) {
  static char ws_buf[1 << 16];
  void* ws = (void*)(((uintptr_t)ws_buf + 255) & ~(uintptr_t)255);
  void* p = (void*)(uintptr_t)(1 << 20); /* never dereferenced: calls must fail first */
  hstu_attn_desc d;

  /* descriptors */
  EXPECT(hstu_attn_fwd(NULL, p, p, 64, p, 64, p, p, p, p, NULL, p, 64, ws, 4096, NULL) ==
         HSTU_ERR_INVALID_ARG);
  d = desc(); d.d_qk = 48;
  EXPECT(hstu_attn_fwd(&d, p, p, 64, p, 64, p, p, p, p, NULL, p, 64, ws, 4096, NULL) ==
         HSTU_ERR_UNSUPPORTED);
  d = desc(); d.T = -1;
  EXPECT(hstu_attn_fwd_workspace_size(&d) == 0);
  d = desc(); d.T = ((int64_t)1 << 31);
  EXPECT(hstu_attn_fwd_workspace_size(&d) == 0);
  d = desc(); d.key_splits = 9;
  EXPECT(hstu_attn_fwd(&d, p, p, 64, p, 64, p, p, p, p, NULL, p, 64, ws, 4096, NULL) ==
         HSTU_ERR_INVALID_ARG);
  d = desc(); d.reuse_plan = 2;
  EXPECT(hstu_attn_fwd(&d, p, p, 64, p, 64, p, p, p, p, NULL, p, 64, ws, 4096, NULL) ==
         HSTU_ERR_INVALID_ARG);
  d = desc(); d.rab_head_stride = 5;
  EXPECT(hstu_attn_bwd_workspace_size(&d) == 0);
  d = desc(); d.norm_len = 0;
  EXPECT(hstu_attn_fwd_workspace_size(&d) == 0);

  /* the largest sizes the checks accept: size arithmetic in 64 bits */
  d = desc(); d.T = ((int64_t)1 << 31) - 1; d.B = 2147483647; d.H = 64; d.d_qk = 128; d.d_v = 128;
  d.max_len = 2147483647; d.key_splits = 8; d.rab_head_stride = 1024;
  d.n_pos_buckets = 1024; d.n_time_buckets = 1024;
  EXPECT(hstu_attn_fwd_workspace_size(&d) > 0);
  EXPECT(hstu_attn_bwd_workspace_size(&d) > 0);
  {
    hstu_layer_desc L;
    memset(&L, 0, sizeof L);
    L.attn = d; L.attn.H = 8; L.D = 1 << 20; L.proj_silu = 1; L.residual = 1; L.ln_eps = 1e-6f;
    EXPECT(hstu_layer_fwd_workspace_size(&L, 1) > 0);
    EXPECT(hstu_layer_bwd_workspace_size(&L) > 0);
    L.D = 12;
    EXPECT(hstu_layer_fwd_workspace_size(&L, 0) == 0);
    EXPECT(hstu_layer_fwd(&L, p, NULL, p, p, NULL, p, NULL, ws, 4096, NULL) != HSTU_OK);
    L.D = 512; L.ln_eps = -1.0f;
    EXPECT(hstu_layer_bwd_workspace_size(&L) == 0);
  }

  /* undersized workspaces are refused before any launch */
  d = desc();
  EXPECT(hstu_attn_fwd(&d, p, p, 64, p, 64, p, p, p, p, NULL, p, 64, ws, 16, NULL) ==
         HSTU_ERR_WORKSPACE);
  EXPECT(hstu_attn_bwd(&d, p, p, 64, p, 64, p, p, p, p, NULL, p, 64, p, p, p, p, p, ws, 16,
                       NULL) == HSTU_ERR_WORKSPACE);

  /* schedule / validation / truncation / MX entry points */
  EXPECT(hstu_schedule_capacity(-1, 4, 128) == 0);
  EXPECT(hstu_schedule_capacity(((int64_t)1 << 40), 2147483647, 1) >= 0);
  EXPECT(hstu_schedule_workspace_size(-1, 10, 128) == 0);
  EXPECT(hstu_schedule(4, 100, NULL, 128, 0, p, p, ws, 4096, NULL) == HSTU_ERR_INVALID_ARG);
  EXPECT(hstu_validate_inputs(4, 100, NULL, NULL, p, NULL) == HSTU_ERR_INVALID_ARG);
  EXPECT(hstu_truncate_offsets(-1, p, NULL, 8, p, NULL) == HSTU_ERR_INVALID_ARG);
  EXPECT(hstu_truncate_gather(4, 100, 10, 7, HSTU_BF16, p, p, p, NULL, p, NULL, NULL) !=
         HSTU_OK);
  EXPECT(hstu_mx_quantize(4, 33, p, 64, p, p, NULL) == HSTU_ERR_INVALID_ARG);
  /* MXFP8 attention operands and scores: extreme sizes are refused on the host */
  EXPECT(hstu_mx_quantize_heads(-1, 2, 64, p, 128, p, 128, (uint32_t*)p, NULL) ==
         HSTU_ERR_INVALID_ARG);
  EXPECT(hstu_mx_quantize_heads(100, 2147483647, 64, p, 128, p, 128, (uint32_t*)p, NULL) ==
         HSTU_ERR_INVALID_ARG);
  EXPECT(hstu_mx_quantize_heads(100, 2, 2147483616, p, 128, p, 128, (uint32_t*)p, NULL) ==
         HSTU_ERR_INVALID_ARG);
  {
    hstu_attn_desc dm = desc();
    dm.d_qk = 64;
    dm.d_v = 64;
    hstu_attn_mx_qk qk;
    qk.q_codes = p;
    qk.k_codes = p;
    qk.ld_codes = 128;
    qk.q_scales = (const uint32_t*)p;
    qk.k_scales = (const uint32_t*)p;
    EXPECT(hstu_attn_fwd_mx(&dm, NULL, p, 128, p, p, p, p, NULL, p, 128, ws, 4096, NULL) ==
           HSTU_ERR_INVALID_ARG);
    qk.ld_codes = -16;
    EXPECT(hstu_attn_fwd_mx(&dm, &qk, p, 128, p, p, p, p, NULL, p, 128, ws, 4096, NULL) ==
           HSTU_ERR_INVALID_ARG);
    qk.ld_codes = 128;
    EXPECT(hstu_attn_fwd_mx(&dm, &qk, p, 128, p, p, p, p, NULL, p, 128, ws, 16, NULL) ==
           HSTU_ERR_WORKSPACE);
    dm.d_qk = 32;
    dm.d_v = 32;
    EXPECT(hstu_attn_fwd_mx(&dm, &qk, p, 128, p, p, p, p, NULL, p, 128, ws, 4096, NULL) ==
           HSTU_ERR_UNSUPPORTED);
    /* the MX layer's workspace with room for MXFP8 scores at a huge T */
    hstu_layer_desc Lm;
    memset(&Lm, 0, sizeof Lm);
    Lm.attn = desc();
    Lm.attn.d_qk = 128;
    Lm.attn.d_v = 128;
    Lm.attn.H = 4;
    Lm.attn.T = (int64_t)1 << 34;
    Lm.D = 512;
    Lm.proj_silu = 1;
    Lm.residual = 1;
    Lm.ln_eps = 1e-6f;
    (void)hstu_layer_fwd_mx_workspace_size(&Lm);
  }
  EXPECT(hstu_set_check_mode(7) == HSTU_ERR_INVALID_ARG);
  EXPECT(hstu_check_mode() == 0);

  /* status texts */
  for (int s = -6; s <= 1; ++s) EXPECT(hstu_status_string((hstu_status)s) != NULL);
  EXPECT(strstr(hstu_version(), "gfx950") != NULL);
  EXPECT(hstu_last_error_site() != NULL);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
