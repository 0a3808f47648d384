/*
 * abi_driver.c -- the host side of the C ABI (include/qsa.h) under
 * AddressSanitizer and UndefinedBehaviorSanitizer (the library's host code is
 * built with them by tests/test_sanitizers.py; device code is not).  Test
 * infrastructure.  Needs no GPU: every call below is answered by host
 * validation and planning before any device call, for valid and invalid
 * configurations of every route, including messages longer than the caller's
 * buffer.  Exit status 0 means clean.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qsa.h"

static int failures = 0;
#define CHECK(c, what)                              \
  do {                                              \
    if (!(c)) {                                     \
      fprintf(stderr, "FAIL: %s\n", what);          \
      ++failures;                                   \
    }                                               \
  } while (0)

static qsa_cfg base(int B, int L, int Hq, int Hkv, int D, int r, int dtype, int msl) {
  qsa_cfg c;
  memset(&c, 0, sizeof c);
  c.batch = B;
  c.q_len = L;
  c.num_q_heads = Hq;
  c.num_kv_heads = Hkv;
  c.head_dim = D;
  c.rotary_dim = r;
  c.rope_theta = 1e7f;
  c.rms_eps = 1e-6f;
  c.dtype = dtype;
  c.max_seq_len = msl;
  c.q_norm_w = (const void *)0x1000;           /* never dereferenced on the host */
  c.k_norm_w = (const void *)0x2000;
  return c;
}

int main(void) {
  char buf[1024], tiny[8];
  const qsa_cfg good[] = {
      base(1, 1, 4, 1, 64, 16, QSA_F32, 33),
      base(1, 1, 16, 4, 256, 64, QSA_BF16, 4097),
      base(8, 4, 24, 2, 256, 64, QSA_BF16, 2052),
      base(64, 1, 16, 4, 256, 64, QSA_BF16, 32769),
      base(1, 2048, 16, 4, 256, 64, QSA_BF16, 32768),
      base(2, 1, 16, 4, 256, 16, QSA_BF16, 300),   /* tile route: r/2 not on whole lanes */
  };
  for (size_t i = 0; i < sizeof good / sizeof good[0]; ++i) {
    qsa_cfg c = good[i];
    const size_t ws = qsa_workspace_size(&c);
    CHECK(ws >= 256, "workspace size of a valid cfg");
    const int n = qsa_describe_plan(&c, buf, sizeof buf);
    CHECK(n > 0 && (size_t)n < sizeof buf && strstr(buf, "route=") != NULL, "plan text");
    CHECK(qsa_describe_plan(&c, tiny, sizeof tiny) == n && strlen(tiny) == sizeof tiny - 1, "plan text truncated");
    for (int k = 1; k <= 65; k += 32) {
      c.force_splits = k;
      CHECK(qsa_workspace_size(&c) >= 256, "forced splits");
    }
    c.force_splits = 0;
    /* a workspace one byte short is refused before any launch */
    qsa_kv_cache kv = {(void *)0x10000, (void *)0x20000, (const int64_t *)0x30000, NULL, 1 << 20};
    c.workspace = (void *)0x40000;
    c.workspace_bytes = ws - 1;
    CHECK(qsa_gated_attention((const void *)0x50000, NULL, NULL, &kv, (const int32_t *)0x60000,
                              (const int32_t *)0x70000, &c, (void *)0x7f0000000000ull) == QSA_ERR_WORKSPACE,
          "short workspace");
    CHECK(strlen(qsa_last_error()) > 0, "message for the last error");
  }
  const qsa_cfg bad[] = {
      base(0, 1, 16, 4, 256, 64, QSA_BF16, 10),
      base(1, 1, 6, 4, 256, 64, QSA_BF16, 10),
      base(1, 1, 16, 4, 96, 32, QSA_BF16, 10),
      base(1, 1, 16, 4, 256, 63, QSA_BF16, 10),
      base(1, 1, 16, 4, 256, 258, QSA_BF16, 10),
      base(1, 1, 16, 4, 256, 64, 7, 10),
      base(1, 4, 16, 4, 256, 64, QSA_BF16, 3),
  };
  for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
    qsa_cfg c = bad[i];
    CHECK(qsa_workspace_size(&c) == 0, "invalid cfg has no workspace size");
    CHECK(qsa_describe_plan(&c, buf, sizeof buf) < 0, "invalid cfg has no plan");
    qsa_kv_cache kv = {(void *)0x10000, (void *)0x20000, (const int64_t *)0x30000, NULL, 1 << 20};
    CHECK(qsa_gated_attention((const void *)0x50000, NULL, NULL, &kv, (const int32_t *)0x60000,
                              (const int32_t *)0x70000, &c, (void *)0x7f0000000000ull) < 0, "invalid cfg refused");
    CHECK(qsa_gated_attention_noalloc((const void *)0x50000, NULL, NULL, &kv, (const int32_t *)0x60000,
                                      (const int32_t *)0x70000, &c, (void *)0x7f0000000000ull) < 0,
          "invalid cfg refused (no-alloc)");
    CHECK(qsa_append_kv((const void *)0x50000, (const void *)0x58000, &kv, (const int32_t *)0x60000,
                        (const int32_t *)0x70000, &c) < 0, "invalid cfg refused (append)");
  }
  CHECK(qsa_workspace_size(NULL) == 0, "NULL cfg");
  CHECK(qsa_gated_attention(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == QSA_ERR_INVALID, "all NULL");
  {
    qsa_cfg c = good[4];                         /* a 12288-row prefill chunk needs more than the no-alloc scratch */
    c.q_len = 12288;
    c.max_seq_len = 12288 + 30720;
    qsa_kv_cache kv = {(void *)0x10000, (void *)0x20000, (const int64_t *)0x30000, NULL, 1 << 20};
    CHECK(qsa_gated_attention_noalloc((const void *)0x50000, NULL, NULL, &kv, (const int32_t *)0x60000,
                                      (const int32_t *)0x70000, &c, (void *)0x7f0000000000ull) ==
              QSA_ERR_WORKSPACE, "no-alloc scratch limit");
  }
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("C ABI host sanitizer run: clean\n");
  return 0;
}
