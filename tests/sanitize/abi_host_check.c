/*
 * Exercises the host side of libmoe's C ABI (include/moe.h) without a GPU,
 * for a build of the library's sources with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code (tests/test_sanitize_cpu.py):
 * problem validation, the size queries over small and very large problems,
 * and every entry point's argument checks (null and misaligned pointers,
 * short workspaces, oversize problems), all of which must return before
 * anything reaches the device. Device pointers are made-up addresses that
 * are never dereferenced. Exit status 0 = every check held and the
 * sanitizers stayed silent.
 */
#include <stdint.h>
#include <stdio.h>

#include "moe.h"

static int fails = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++fails;                                                     \
    }                                                              \
  } while (0)

#define FAKE(a) ((void*)(uintptr_t)(a))

static moe_problem prob(int64_t T, int E, int k, int d, int h, int hs, int dt, int bm, int cap) {
  moe_problem p = {T, E, k, d, h, hs, dt, bm, cap};
  return p;
}

int main(void) {
  CHECK(moe_check_problem(NULL) == MOE_ERR_INVALID);
  CHECK(moe_status_string(MOE_ERR_TOO_LARGE) != NULL && moe_status_string(12345) != NULL);
  CHECK(moe_version() != NULL);
  /* size queries over a spread of problems, up to the largest supported ones */
  const int64_t toks[] = {0, 1, 4096, 131072, (int64_t)1 << 27, ((int64_t)1 << 31) / 64 - 1};
  const int Es[] = {1, 8, 64}, ds[] = {128, 512, 8192}, hs_[] = {0, 1024};
  for (unsigned a = 0; a < sizeof(toks) / sizeof(toks[0]); ++a)
    for (unsigned b = 0; b < 3; ++b)
      for (unsigned c = 0; c < 3; ++c)
        for (unsigned e = 0; e < 2; ++e)
          for (int dt = 0; dt < 2; ++dt) {
            const int E = Es[b], k = E < 8 ? E : 8;
            moe_problem p = prob(toks[a], E, k, ds[c], 256, hs_[e], dt, 128, 0);
            const int st = moe_check_problem(&p);
            CHECK(st == MOE_OK || st == MOE_ERR_UNSUPPORTED);
            if (st != MOE_OK) continue;
            CHECK(moe_param_count(&p) > 0);
            CHECK(moe_max_tiles(&p) >= E);
            CHECK(moe_workspace_bytes(&p, 0) >= 256 && moe_workspace_bytes(&p, 1) >= 256);
            (void)moe_saved_bytes(&p);
            for (int disp = 0; disp < 3; ++disp)
              CHECK(moe_forward_workspace_bytes(&p, disp, disp & 1) >= 256);
            CHECK(moe_forward_workspace_bytes(&p, 3, 0) == 0);
          }
  /* invalid and unsupported problems */
  moe_problem bad[] = {prob(-1, 8, 2, 256, 128, 0, 1, 64, 0), prob(10, 0, 1, 256, 128, 0, 1, 64, 0),
                       prob(10, 8, 9, 256, 128, 0, 1, 64, 0), prob(10, 8, 2, 256, 128, 0, 7, 64, 0),
                       prob(10, 8, 2, 256, 128, -64, 1, 64, 0), prob(10, 8, 2, 256, 128, 0, 1, 64, -1),
                       prob(10, 65, 2, 256, 128, 0, 1, 64, 0), prob(10, 8, 2, 250, 128, 0, 1, 64, 0),
                       prob(10, 8, 2, 256, 100, 0, 1, 64, 0), prob(10, 8, 2, 256, 128, 0, 1, 48, 0),
                       prob((int64_t)1 << 30, 8, 2, 256, 128, 0, 1, 64, 0),
                       prob(INT64_MAX / 2, 8, 8, 256, 128, 0, 1, 64, 0)};
  for (unsigned i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
    CHECK(moe_check_problem(&bad[i]) != MOE_OK);
    CHECK(moe_workspace_bytes(&bad[i], 1) == 0 && moe_saved_bytes(&bad[i]) == 0);
    CHECK(moe_max_tiles(&bad[i]) == 0 && moe_param_count(&bad[i]) == -1);
    moe_routing r0 = {0};
    CHECK(moe_route(&bad[i], FAKE(0x1000), FAKE(0x1000), &r0, NULL) != MOE_OK);
    CHECK(moe_permute_static(&bad[i], &r0, NULL) != MOE_OK);
  }
  /* argument checks of every entry point (nothing is enqueued) */
  moe_problem p = prob(100, 8, 2, 256, 128, 128, MOE_BF16, 64, 0);
  moe_routing r = {FAKE(0x10000000), FAKE(0x10100000), FAKE(0x10200000), FAKE(0x10300000),
                   FAKE(0x10400000), FAKE(0x10500000), FAKE(0x10600000)};
  moe_weights w = {FAKE(0x20000000), FAKE(0x20100000), FAKE(0x20200000), FAKE(0x20300000),
                   FAKE(0x20400000), FAKE(0x20500000), FAKE(0x20600000)};
  moe_grads g = {FAKE(0x30000000), FAKE(0x30100000), FAKE(0x30200000), FAKE(0x30300000),
                 FAKE(0x30400000), FAKE(0x30500000), FAKE(0x30600000)};
  void* x = FAKE(0x40000000);
  void* ws = FAKE(0x50000000);
  const size_t need = moe_workspace_bytes(&p, 1);
  CHECK(moe_route(&p, NULL, w.w_router, &r, NULL) == MOE_ERR_INVALID);
  CHECK(moe_route(&p, FAKE(0x40000008), w.w_router, &r, NULL) == MOE_ERR_INVALID);
  CHECK(moe_route(&p, x, w.w_router, NULL, NULL) == MOE_ERR_INVALID);
  CHECK(moe_permute(&p, &r, ws, 0, NULL) == MOE_ERR_WORKSPACE);
  CHECK(moe_permute(&p, &r, FAKE(0x50000010), need, NULL) == MOE_ERR_INVALID);
  moe_routing r_bad = r;
  r_bad.perm = NULL;
  CHECK(moe_permute(&p, &r_bad, ws, need, NULL) == MOE_ERR_INVALID);
  CHECK(moe_permute_static(&p, &r_bad, NULL) == MOE_ERR_INVALID);
  moe_problem huge = prob(((int64_t)1 << 24) / 8 + 1, 64, 8, 128, 64, 0, MOE_BF16, 256, 0);
  CHECK(moe_permute_static(&huge, &r, NULL) == MOE_ERR_TOO_LARGE);
  CHECK(moe_ffn_fwd(&p, x, &w, &r, FAKE(0x60000000), FAKE(0x61000000), NULL, ws, 16, NULL) ==
        MOE_ERR_WORKSPACE);
  CHECK(moe_ffn_fwd(&p, x, &w, &r, FAKE(0x60000000), NULL, NULL, ws, need, NULL) ==
        MOE_ERR_INVALID);
  CHECK(moe_ffn_fwd(&p, x, &w, &r, FAKE(0x60000000), FAKE(0x61000000), FAKE(0x62000010), ws, need,
                    NULL) == MOE_ERR_INVALID);
  CHECK(moe_combine(&p, NULL, &r, NULL, FAKE(0x63000000), NULL) == MOE_ERR_INVALID);
  CHECK(moe_combine(&p, FAKE(0x60000000), &r, FAKE(0x61000004), FAKE(0x63000000), NULL) ==
        MOE_ERR_INVALID);
  CHECK(moe_forward(&p, 9, x, &w, &r, FAKE(0x60000000), NULL, FAKE(0x63000000), ws, need, NULL,
                    NULL) ==
        MOE_ERR_INVALID);
  CHECK(moe_forward(&p, MOE_DISPATCH_GATHER, x, &w, &r, FAKE(0x60000000), NULL, FAKE(0x63000000),
                    ws, 16, NULL, NULL) == MOE_ERR_WORKSPACE);
  moe_weights w_noshared = w;
  w_noshared.ws_up = NULL;
  CHECK(moe_forward(&p, MOE_DISPATCH_FUSED_GSUM, x, &w_noshared, &r, FAKE(0x60000000), NULL,
                    FAKE(0x63000000), ws, need, NULL, NULL) == MOE_ERR_INVALID);
  moe_problem p_h = prob(100, 8, 2, 256, 192, 0, MOE_BF16, 64, 0);
  CHECK(moe_bwd(&p_h, x, &w, &r, FAKE(0x60000000), FAKE(0x70000000), FAKE(0x71000000),
                FAKE(0x72000000), &g, ws, need, NULL, NULL) == MOE_ERR_UNSUPPORTED);
  CHECK(moe_bwd(&p, x, &w, &r, FAKE(0x60000000), FAKE(0x70000000), FAKE(0x71000000),
                FAKE(0x72000000), NULL, ws, need, NULL, NULL) == MOE_ERR_INVALID);
  CHECK(moe_bwd(&p, x, &w, &r, FAKE(0x60000000), FAKE(0x70000010), FAKE(0x71000000),
                FAKE(0x72000000), &g, ws, need, NULL, NULL) == MOE_ERR_INVALID);
  CHECK(moe_bwd(&p, x, &w, &r, FAKE(0x60000000), FAKE(0x70000000), FAKE(0x71000000),
                FAKE(0x72000000), &g, ws, 16, NULL, NULL) == MOE_ERR_WORKSPACE);
  /* zero tokens: successful no-ops that never touch their pointers */
  moe_problem z = prob(0, 8, 2, 256, 128, 0, MOE_BF16, 64, 0);
  CHECK(moe_route(&z, NULL, NULL, NULL, NULL) == MOE_OK);
  CHECK(moe_permute(&z, NULL, NULL, 0, NULL) == MOE_OK);
  CHECK(moe_permute_static(&z, NULL, NULL) == MOE_OK);
  CHECK(moe_ffn_fwd(&z, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == MOE_OK);
  CHECK(moe_combine(&z, NULL, NULL, NULL, NULL, NULL) == MOE_OK);
  CHECK(moe_forward(&z, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL) == MOE_OK);
  char buf[8];
  CHECK(moe_trace_summary(NULL, 0) == MOE_ERR_INVALID);
  CHECK(moe_trace_summary(buf, 1) == MOE_ERR_INVALID || moe_trace_summary(buf, 1) == MOE_OK);
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  else printf("ABI host sanitizer run clean\n");
  return fails ? 1 : 0;
}
