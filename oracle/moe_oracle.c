/*
 * CPU oracle for the dropless top-k Mixture-of-Experts layer (forward and
 * train-step gradients).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header or table with the HIP library and includes nothing from it.
 *
 * What is computed follows the benchmark pages (probjax kernel_gmm_gpu.json,
 * gpu_nn.json, gpu_moe_h100.json):
 *   - gpu_moe_h100.json, header "description": a dropless MoE layer, forward
 *     and a train step taking value and gradient with respect to the
 *     parameters and the input;
 *   - kernel_gmm_gpu.json, "pieces" suite records: the stages route ->
 *     sort_permute -> experts_grouped_swiglu -> unpermute_combine;
 *   - gpu_nn.json, "moe" suite, "params" field: 12,587,008 parameters at
 *     E=8, d_model 512, d_hidden 1024, which is 3*E*d*h + d*E, so there are no
 *     biases and the router is one bias-free [d,E] matrix;
 *   - kernel_gmm_gpu.json "pieces" records, "xla_arg_mb": the router matrix
 *     and the combine weights are fp32 even when tokens are bf16.
 * The routing rule (softmax over the E logits, keep the top_k largest, the
 * lower expert index winning ties, renormalise the kept weights), the gated
 * expert (SiLU(x W_gate) * (x W_up)) W_down, the always-on shared expert and
 * the loss sum(out * G) are the layer's definition for these workloads.
 *
 * Arithmetic: every floating-point result is computed in double from the
 * stored input values (bf16 inputs arrive already widened exactly to fp32),
 * except the router logits, which follow one fixed fp32 order (see
 * oracle_route) so that expert choices can be compared exactly.
 *
 *
 * Capacity routing (kernel_gmm_gpu.json records with "routing": "capacity";
 * the pages give neither the capacity nor the drop rule, so this is the
 * reading adopted): each expert takes at most `capacity` token-slots, the
 * first ones in flat slot order t*k+i; a dropped slot contributes nothing
 * to the output and no gradient to its expert's weights, the kept weights
 * are not renormalised, and the router gradient still flows through every
 * selected slot's weight. capacity 0 means dropless.
 *
 * Parity pins (all in the CPU test suite): dense every-expert-masked brute
 * force, finite differences, closed-form special cases (all-zero router,
 * k == E, E == k == 1, identical experts, k == 1), the constructed
 * permutation, tile invariants and the pages' parameter count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_API __attribute__((visibility("default")))

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

ORACLE_API int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Parameter count: three [d,h] / [h,d] matrices per expert, one bias-free
 * router [d,E], three shared matrices when a shared expert exists. */
ORACLE_API int64_t oracle_param_count(int64_t E, int64_t d, int64_t h, int64_t hs) {
  return 3 * E * d * h + d * E + 3 * d * hs;
}

/* ---------------------------------------------------------------- routing */

typedef struct {
  float v;
  int e;
} scored;

/* (value descending, expert index ascending): a total order, so qsort's
 * instability cannot matter. */
static int cmp_scored(const void* pa, const void* pb) {
  const scored* a = (const scored*)pa;
  const scored* b = (const scored*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->e < b->e) ? -1 : (a->e > b->e);
}

/*
 * Router logits, top-k selection and renormalised combine weights.
 *   logits[t,e]: fp32, acc = +0.0f; for j = 0..d-1: acc = fmaf(x[t,j], wr[j,e], acc)
 *   topk_idx[t,i]: the i-th expert in (logit desc, index asc) order, i < k
 *   topk_w[t,i] (double): exp(l_i - l_0) / sum_j exp(l_j - l_0) over the k kept
 * logits may be NULL. Returns 0.
 */
ORACLE_API int oracle_route(int64_t T, int d, int E, int k, const float* x, const float* wr,
                            float* logits, int32_t* topk_idx, double* topk_w, int nthreads) {
  set_threads(nthreads);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    scored* s = (scored*)malloc(sizeof(scored) * (size_t)E);
    for (int e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int j = 0; j < d; ++j) acc = fmaf(x[t * d + j], wr[(int64_t)j * E + e], acc);
      s[e].v = acc;
      s[e].e = e;
      if (logits) logits[t * E + e] = acc;
    }
    qsort(s, (size_t)E, sizeof(scored), cmp_scored);
    double m = (double)s[0].v, z = 0.0;
    for (int i = 0; i < k; ++i) z += exp((double)s[i].v - m);
    for (int i = 0; i < k; ++i) {
      topk_idx[t * k + i] = s[i].e;
      topk_w[t * k + i] = exp((double)s[i].v - m) / z;
    }
    free(s);
  }
  return 0;
}

/*
 * Stable grouping of the T*k token-slots by expert, and the block_m tile
 * schedule ("sort_permute" piece; block_m field of the kernel_gmm_gpu.json
 * config blocks).
 *   counts[e]      = number of slots (t,i) with topk_idx[t,i] == e
 *   offsets[e]     = sum of counts[e'] for e' < e; offsets[E] = T*k
 *   perm[slot]     = flat slot t*k+i placed at sorted position slot, where the
 *                    slots of one expert keep ascending flat order
 *   inv_perm[flat] = its sorted position, or -1 when capacity > 0 and the
 *                    slot is not among the first `capacity` of its expert
 *   tiles[3*n..]   = (expert, first sorted row, rows) for each block_m-row
 *                    piece of each expert's kept rows, experts ascending
 * Returns the number of tiles, or -1 on an out-of-range expert index.
 */
ORACLE_API int64_t oracle_permute(int64_t T, int k, int E, int bm, int capacity,
                                  const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                                  int32_t* perm, int32_t* inv_perm, int32_t* tiles) {
  const int64_t S = T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t s = 0; s < S; ++s) {
    int e = topk_idx[s];
    if (e < 0 || e >= E) return -1;
    counts[e]++;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* next = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t s = 0; s < S; ++s) {
    int e = topk_idx[s];
    int32_t rank = next[e]++;
    int32_t pos = offsets[e] + rank;
    perm[pos] = (int32_t)s;
    inv_perm[s] = (capacity > 0 && rank >= capacity) ? -1 : pos;
  }
  free(next);
  int64_t n = 0;
  for (int e = 0; e < E; ++e) {
    int32_t kept = (capacity > 0 && counts[e] > capacity) ? capacity : counts[e];
    for (int32_t r = 0; r < kept; r += bm) {
      int32_t rows = kept - r < bm ? kept - r : bm;
      if (tiles) {
        tiles[3 * n + 0] = e;
        tiles[3 * n + 1] = offsets[e] + r;
        tiles[3 * n + 2] = rows;
      }
      ++n;
    }
  }
  return n;
}

/* ---------------------------------------------------------- expert FFN */

static double silu(double a) { return a / (1.0 + exp(-a)); }
static double sigmoid(double a) { return 1.0 / (1.0 + exp(-a)); }

/* One gated FFN on one token row: a = x Wg, b = x Wu (both [d,h] row-major),
 * g = SiLU(a) * b, y = g Wd ([h,d] row-major). a, b, g have h entries,
 * y has d. */
static void ffn_row(int d, int h, const float* xr, const float* wg, const float* wu,
                    const float* wd, double* a, double* b, double* g, double* y) {
  for (int c = 0; c < h; ++c) a[c] = b[c] = 0.0;
  for (int j = 0; j < d; ++j) {
    double xj = (double)xr[j];
    const float* rg = wg + (int64_t)j * h;
    const float* ru = wu + (int64_t)j * h;
    for (int c = 0; c < h; ++c) {
      a[c] += xj * (double)rg[c];
      b[c] += xj * (double)ru[c];
    }
  }
  for (int c = 0; c < h; ++c) g[c] = silu(a[c]) * b[c];
  for (int j = 0; j < d; ++j) y[j] = 0.0;
  for (int c = 0; c < h; ++c) {
    double gc = g[c];
    const float* rd = wd + (int64_t)c * d;
    for (int j = 0; j < d; ++j) y[j] += gc * (double)rd[j];
  }
}

/*
 * Forward output rows.
 *   out[r,:] = sum_i topk_w[t,i] * FFN_{topk_idx[t,i]}(x[t]) + FFN_shared(x[t])
 * for t = rows[r] (rows == NULL means t = r for r < nrows). The shared term is
 * present when hs > 0. When y_slots is non-NULL, y_slots[r*k+i,:] receives
 * the unweighted expert output of selection i (the sorted expert outputs,
 * indexed by flat slot). Weights of expert e: wg + e*d*h, wu + e*d*h,
 * wd + e*h*d. keep (T*k flags, NULL = all kept): a slot with keep == 0 was
 * dropped by capacity routing and contributes nothing (its y_slots row is 0).
 */
ORACLE_API int oracle_forward_rows(int64_t nrows, const int64_t* rows, int d, int E, int k, int h,
                                   int hs, const float* x, const float* wg, const float* wu,
                                   const float* wd, const float* wsg, const float* wsu,
                                   const float* wsd, const int32_t* topk_idx,
                                   const double* topk_w, const uint8_t* keep, double* out,
                                   double* y_slots, int nthreads) {
  (void)E;
  set_threads(nthreads);
  int hmax = h > hs ? h : hs;
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)hmax);
    double* b = (double*)malloc(sizeof(double) * (size_t)hmax);
    double* g = (double*)malloc(sizeof(double) * (size_t)hmax);
    double* y = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
      int64_t t = rows ? rows[r] : r;
      const float* xr = x + t * d;
      double* o = out + r * d;
      for (int j = 0; j < d; ++j) o[j] = 0.0;
      for (int i = 0; i < k; ++i) {
        int64_t e = topk_idx[t * k + i];
        double w = topk_w[t * k + i];
        if (keep && !keep[t * k + i]) {
          if (y_slots) memset(y_slots + (r * k + i) * d, 0, sizeof(double) * (size_t)d);
          continue;
        }
        ffn_row(d, h, xr, wg + e * d * h, wu + e * d * h, wd + e * h * d, a, b, g, y);
        for (int j = 0; j < d; ++j) o[j] += w * y[j];
        if (y_slots) memcpy(y_slots + (r * k + i) * d, y, sizeof(double) * (size_t)d);
      }
      if (hs > 0) {
        ffn_row(d, hs, xr, wsg, wsu, wsd, a, b, g, y);
        for (int j = 0; j < d; ++j) o[j] += y[j];
      }
    }
    free(a);
    free(b);
    free(g);
    free(y);
  }
  return 0;
}

/* Backward of one gated FFN row for the upstream gradient dy (d entries):
 * returns dg-derived da, db (h entries) and accumulates dx += da Wg^T + db Wu^T.
 * SiLU'(a) = sigmoid(a) (1 + a (1 - sigmoid(a))). */
static void ffn_row_bwd(int d, int h, const float* wg, const float* wu, const float* wd,
                        const double* a, const double* b, const double* dy, double* da,
                        double* db, double* dx) {
  for (int c = 0; c < h; ++c) {
    const float* rd = wd + (int64_t)c * d;
    double dg = 0.0;
    for (int j = 0; j < d; ++j) dg += (double)rd[j] * dy[j];
    double s = sigmoid(a[c]);
    da[c] = dg * b[c] * s * (1.0 + a[c] * (1.0 - s));
    db[c] = dg * a[c] * s;
  }
  for (int j = 0; j < d; ++j) {
    const float* rg = wg + (int64_t)j * h;
    const float* ru = wu + (int64_t)j * h;
    double acc = 0.0;
    for (int c = 0; c < h; ++c) acc += da[c] * (double)rg[c] + db[c] * (double)ru[c];
    dx[j] += acc;
  }
}

/*
 * Train-step gradients of L = sum(out * G) with the top-k selection held
 * fixed (gradient reaches the router through the renormalised weights):
 *   dy_i = w_i G_t;  dw_i = <G_t, y_i>
 *   dW_down[e] += g_i^T dy_i;  da, db from dg = dy_i W_down[e]^T
 *   dW_gate[e] += x_t^T da;  dW_up[e] += x_t^T db
 *   dx_t += da W_gate[e]^T + db W_up[e]^T
 *   dl_i = w_i (dw_i - sum_j w_j dw_j) on the kept experts, 0 elsewhere
 *   dW_r += x_t^T dl;  dx_t += dl W_r^T
 *   shared expert: the same steps with weight 1.
 * A slot dropped by capacity routing (keep[s] == 0; keep NULL = all kept)
 * has y_i = 0: dw_i = 0, no expert-weight or expert-path input gradient,
 * while dl_i = w_i (0 - sum_j w_j dw_j) still reaches the router.
 * All outputs are double and fully overwritten; the shared ones are touched
 * only when hs > 0. Weight gradients of expert e are reduced over tokens in
 * ascending token order.
 */
ORACLE_API int oracle_backward(int64_t T, int d, int E, int k, int h, int hs, const float* x,
                               const float* wr, const float* wg, const float* wu, const float* wd,
                               const float* wsg, const float* wsu, const float* wsd,
                               const float* G, const int32_t* topk_idx, const double* topk_w,
                               const uint8_t* keep, double* dx, double* dwr, double* dwg,
                               double* dwu, double* dwd, double* dwsg, double* dwsu, double* dwsd,
                               int nthreads) {
  set_threads(nthreads);
  const int64_t S = T * k;
  /* Per-slot and per-token intermediates (phase 1, token-parallel). */
  double* G_a = (double*)malloc(sizeof(double) * (size_t)(S * h)); /* gate pre-activation */
  double* G_b = (double*)malloc(sizeof(double) * (size_t)(S * h)); /* up pre-activation */
  double* Dda = (double*)malloc(sizeof(double) * (size_t)(S * h));
  double* Ddb = (double*)malloc(sizeof(double) * (size_t)(S * h));
  double* dl = (double*)malloc(sizeof(double) * (size_t)(S)); /* router grad per slot */
  double *Sa = NULL, *Sb = NULL, *Sda = NULL, *Sdb = NULL;
  if (hs > 0) {
    Sa = (double*)malloc(sizeof(double) * (size_t)(T * hs));
    Sb = (double*)malloc(sizeof(double) * (size_t)(T * hs));
    Sda = (double*)malloc(sizeof(double) * (size_t)(T * hs));
    Sdb = (double*)malloc(sizeof(double) * (size_t)(T * hs));
  }
  int hmax = h > hs ? h : hs;
#pragma omp parallel
  {
    double* g = (double*)malloc(sizeof(double) * (size_t)hmax);
    double* y = (double*)malloc(sizeof(double) * (size_t)d);
    double* dy = (double*)malloc(sizeof(double) * (size_t)d);
    double* dw = (double*)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(dynamic, 16)
    for (int64_t t = 0; t < T; ++t) {
      const float* xr = x + t * d;
      const float* Gt = G + t * d;
      double* dxt = dx + t * d;
      for (int j = 0; j < d; ++j) dxt[j] = 0.0;
      double sdw = 0.0;
      for (int i = 0; i < k; ++i) {
        int64_t s = t * k + i;
        int64_t e = topk_idx[s];
        double w = topk_w[s];
        double* a = G_a + s * h;
        double* b = G_b + s * h;
        if (keep && !keep[s]) {
          dw[i] = 0.0;
          continue;
        }
        ffn_row(d, h, xr, wg + e * d * h, wu + e * d * h, wd + e * h * d, a, b, g, y);
        double acc = 0.0;
        for (int j = 0; j < d; ++j) {
          acc += (double)Gt[j] * y[j];
          dy[j] = w * (double)Gt[j];
        }
        dw[i] = acc;
        sdw += w * acc;
        ffn_row_bwd(d, h, wg + e * d * h, wu + e * d * h, wd + e * h * d, a, b, dy, Dda + s * h,
                    Ddb + s * h, dxt);
      }
      for (int i = 0; i < k; ++i) {
        int64_t s = t * k + i;
        int64_t e = topk_idx[s];
        double v = topk_w[s] * (dw[i] - sdw);
        dl[s] = v;
        for (int j = 0; j < d; ++j) dxt[j] += v * (double)wr[(int64_t)j * E + e];
      }
      if (hs > 0) {
        double* a = Sa + t * hs;
        double* b = Sb + t * hs;
        ffn_row(d, hs, xr, wsg, wsu, wsd, a, b, g, y);
        for (int j = 0; j < d; ++j) dy[j] = (double)Gt[j];
        ffn_row_bwd(d, hs, wsg, wsu, wsd, a, b, dy, Sda + t * hs, Sdb + t * hs, dxt);
      }
    }
    free(g);
    free(y);
    free(dy);
    free(dw);
  }

  /* Phase 2: weight gradients, each output element reduced over tokens in
   * ascending order (parallel over experts / rows only). */
  memset(dwr, 0, sizeof(double) * (size_t)d * E);
#pragma omp parallel for schedule(static)
  for (int j = 0; j < d; ++j) {
    for (int64_t t = 0; t < T; ++t) {
      double xj = (double)x[t * d + j];
      for (int i = 0; i < k; ++i) {
        int64_t s = t * k + i;
        dwr[(int64_t)j * E + topk_idx[s]] += xj * dl[s];
      }
    }
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int e = 0; e < E; ++e) {
    double* pg = dwg + (int64_t)e * d * h;
    double* pu = dwu + (int64_t)e * d * h;
    double* pd = dwd + (int64_t)e * h * d;
    memset(pg, 0, sizeof(double) * (size_t)d * h);
    memset(pu, 0, sizeof(double) * (size_t)d * h);
    memset(pd, 0, sizeof(double) * (size_t)h * d);
    double* gv = (double*)malloc(sizeof(double) * (size_t)h);
    for (int64_t t = 0; t < T; ++t) {
      for (int i = 0; i < k; ++i) {
        int64_t s = t * k + i;
        if (topk_idx[s] != e || (keep && !keep[s])) continue;
        const float* xr = x + t * d;
        const float* Gt = G + t * d;
        double w = topk_w[s];
        const double* a = G_a + s * h;
        const double* b = G_b + s * h;
        for (int c = 0; c < h; ++c) gv[c] = silu(a[c]) * b[c];
        for (int c = 0; c < h; ++c)
          for (int j = 0; j < d; ++j) pd[(int64_t)c * d + j] += gv[c] * w * (double)Gt[j];
        const double* da = Dda + s * h;
        const double* db = Ddb + s * h;
        for (int j = 0; j < d; ++j) {
          double xj = (double)xr[j];
          for (int c = 0; c < h; ++c) {
            pg[(int64_t)j * h + c] += xj * da[c];
            pu[(int64_t)j * h + c] += xj * db[c];
          }
        }
      }
    }
    free(gv);
  }
  if (hs > 0) {
    memset(dwsg, 0, sizeof(double) * (size_t)d * hs);
    memset(dwsu, 0, sizeof(double) * (size_t)d * hs);
    memset(dwsd, 0, sizeof(double) * (size_t)hs * d);
#pragma omp parallel for schedule(dynamic, 4)
    for (int j = 0; j < d; ++j) {
      for (int64_t t = 0; t < T; ++t) {
        double xj = (double)x[t * d + j];
        const double* da = Sda + t * hs;
        const double* db = Sdb + t * hs;
        for (int c = 0; c < hs; ++c) {
          dwsg[(int64_t)j * hs + c] += xj * da[c];
          dwsu[(int64_t)j * hs + c] += xj * db[c];
        }
      }
    }
#pragma omp parallel for schedule(dynamic, 4)
    for (int c = 0; c < hs; ++c) {
      for (int64_t t = 0; t < T; ++t) {
        double gc = silu(Sa[t * hs + c]) * Sb[t * hs + c];
        const float* Gt = G + t * d;
        for (int j = 0; j < d; ++j) dwsd[(int64_t)c * d + j] += gc * (double)Gt[j];
      }
    }
  }
  free(G_a);
  free(G_b);
  free(Dda);
  free(Ddb);
  free(dl);
  free(Sa);
  free(Sb);
  free(Sda);
  free(Sdb);
  return 0;
}
