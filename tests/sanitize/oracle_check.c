/*
 * Drives every entry point of the CPU oracle (oracle/moe_oracle.c) on small
 * problems, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitize_cpu.py). Input values come from a small linear
 * congruential sequence: only memory accesses and undefined behaviour are
 * checked here, plus a few invariants of the routing state (each expert's
 * rows contiguous, the permutation a bijection, tiles covering the kept
 * rows). Exit status 0 = clean.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_max_threads(void);
int64_t oracle_param_count(int64_t E, int64_t d, int64_t h, int64_t hs);
int oracle_route(int64_t T, int d, int E, int k, const float* x, const float* wr, float* logits,
                 int32_t* topk_idx, double* topk_w, int nthreads);
int64_t oracle_permute(int64_t T, int k, int E, int bm, int capacity, const int32_t* topk_idx,
                       int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                       int32_t* tiles);
int oracle_forward_rows(int64_t nrows, const int64_t* rows, int d, int E, int k, int h, int hs,
                        const float* x, const float* wg, const float* wu, const float* wd,
                        const float* wsg, const float* wsu, const float* wsd,
                        const int32_t* topk_idx, const double* topk_w, const uint8_t* keep,
                        double* out, double* y_slots, int nthreads);
int oracle_backward(int64_t T, int d, int E, int k, int h, int hs, const float* x,
                    const float* wr, const float* wg, const float* wu, const float* wd,
                    const float* wsg, const float* wsu, const float* wsd, const float* G,
                    const int32_t* topk_idx, const double* topk_w, const uint8_t* keep,
                    double* dx, double* dwr, double* dwg, double* dwu, double* dwd, double* dwsg,
                    double* dwsu, double* dwsd, int nthreads);

static uint64_t lcg = 12345;
static float val(float scale) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return scale * ((float)((lcg >> 40) & 0xffff) / 32768.0f - 1.0f);
}
static float* fill(size_t n, float scale) {
  float* a = (float*)malloc(n * sizeof(float) + 1);
  for (size_t i = 0; i < n; ++i) a[i] = val(scale);
  return a;
}
static int fails = 0;
#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++fails;                                                \
    }                                                         \
  } while (0)

static void run(int64_t T, int d, int E, int k, int h, int hs, int bm, int cap, int nthreads) {
  const int64_t S = T * k;
  float* x = fill((size_t)T * d, 1.0f);
  float* wr = fill((size_t)d * E, 0.1f);
  float* wg = fill((size_t)E * d * h, 0.1f);
  float* wu = fill((size_t)E * d * h, 0.1f);
  float* wd = fill((size_t)E * h * d, 0.1f);
  float* wsg = hs ? fill((size_t)d * hs, 0.1f) : NULL;
  float* wsu = hs ? fill((size_t)d * hs, 0.1f) : NULL;
  float* wsd = hs ? fill((size_t)hs * d, 0.1f) : NULL;
  float* G = fill((size_t)T * d, 1.0f);
  float* logits = (float*)malloc(sizeof(float) * (size_t)(T * E) + 1);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)S + 1);
  double* w = (double*)malloc(sizeof(double) * (size_t)S + 1);
  CHECK(oracle_route(T, d, E, k, x, wr, logits, idx, w, nthreads) == 0);
  for (int64_t s = 0; s < S; ++s) CHECK(idx[s] >= 0 && idx[s] < E);
  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)S + 1);
  int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)S + 1);
  const int64_t max_tiles = (S + bm - 1) / bm + E;
  int32_t* tiles = (int32_t*)malloc(sizeof(int32_t) * (size_t)(3 * max_tiles));
  const int64_t nt = oracle_permute(T, k, E, bm, cap, idx, counts, offsets, perm, inv, tiles);
  CHECK(nt >= 0 && nt <= max_tiles);
  CHECK(offsets[0] == 0 && offsets[E] == S);
  uint8_t* seen = (uint8_t*)calloc((size_t)S + 1, 1);
  for (int64_t j = 0; j < S; ++j) {
    CHECK(perm[j] >= 0 && perm[j] < S);
    if (perm[j] >= 0 && perm[j] < S) seen[perm[j]]++;
  }
  for (int64_t s = 0; s < S; ++s) CHECK(seen[s] == 1);
  int64_t covered = 0;
  for (int64_t n = 0; n < nt; ++n) covered += tiles[3 * n + 2];
  int64_t kept = 0;
  uint8_t* keep = (uint8_t*)malloc((size_t)S + 1);
  for (int64_t s = 0; s < S; ++s) {
    keep[s] = inv[s] >= 0;
    kept += keep[s];
  }
  CHECK(covered == kept);
  CHECK(cap > 0 || kept == S);
  /* every token, then a subset of rows, with the per-slot outputs */
  double* out = (double*)malloc(sizeof(double) * (size_t)((T > 3 ? T : 3) * d) + 1);
  double* y = (double*)malloc(sizeof(double) * (size_t)(S * d) + 1);
  CHECK(oracle_forward_rows(T, NULL, d, E, k, h, hs, x, wg, wu, wd, wsg, wsu, wsd, idx, w,
                            cap ? keep : NULL, out, y, nthreads) == 0);
  if (T > 0) {
    int64_t rows[3] = {T - 1, 0, T / 2};
    CHECK(oracle_forward_rows(3, rows, d, E, k, h, hs, x, wg, wu, wd, wsg, wsu, wsd, idx, w, NULL,
                              out, NULL, nthreads) == 0);
  }
  double* dx = (double*)malloc(sizeof(double) * (size_t)(T * d) + 1);
  double* dwr = (double*)malloc(sizeof(double) * (size_t)(d * E));
  double* dwg = (double*)malloc(sizeof(double) * (size_t)E * d * h);
  double* dwu = (double*)malloc(sizeof(double) * (size_t)E * d * h);
  double* dwd = (double*)malloc(sizeof(double) * (size_t)E * h * d);
  double* dwsg = hs ? (double*)malloc(sizeof(double) * (size_t)d * hs) : NULL;
  double* dwsu = hs ? (double*)malloc(sizeof(double) * (size_t)d * hs) : NULL;
  double* dwsd = hs ? (double*)malloc(sizeof(double) * (size_t)hs * d) : NULL;
  CHECK(oracle_backward(T, d, E, k, h, hs, x, wr, wg, wu, wd, wsg, wsu, wsd, G, idx, w,
                        cap ? keep : NULL, dx, dwr, dwg, dwu, dwd, dwsg, dwsu, dwsd,
                        nthreads) == 0);
  free(x); free(wr); free(wg); free(wu); free(wd); free(wsg); free(wsu); free(wsd); free(G);
  free(logits); free(idx); free(w); free(counts); free(offsets); free(perm); free(inv);
  free(tiles); free(seen); free(keep); free(out); free(y); free(dx); free(dwr); free(dwg);
  free(dwu); free(dwd); free(dwsg); free(dwsu); free(dwsd);
}

int main(void) {
  CHECK(oracle_param_count(8, 512, 1024, 0) == 12587008);
  CHECK(oracle_max_threads() >= 1);
  run(37, 16, 4, 2, 8, 0, 4, 0, 1);
  run(37, 16, 4, 2, 8, 8, 4, 5, 2);   /* shared expert, capacity drops */
  run(1, 8, 3, 3, 4, 4, 32, 0, 1);    /* one token, k = E */
  run(50, 8, 1, 1, 4, 0, 8, 0, 1);    /* one expert */
  run(64, 24, 8, 8, 6, 6, 16, 3, 0);  /* k = E, tight capacity, all threads */
  run(0, 8, 4, 2, 4, 0, 4, 0, 1);     /* no tokens */
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  else printf("oracle sanitizer run clean\n");
  return fails ? 1 : 0;
}
