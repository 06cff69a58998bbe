/*
 * A plain C caller of libcce (no Python, no torch): device memory and a
 * stream from the HIP runtime, every entry point called through cce.h.
 *
 * The check uses a closed form instead of an oracle: with a zero classifier
 * (c = 0) every logit is 0, so LSE_i = ln V and loss_i = ln V on every row,
 * and the mean loss is ln V (the tirogla "Loss functions" page checks
 * exactly this value, ln 1000, for V = 1000).  The softmax is 1/V
 * everywhere, above the 2^-12 filter threshold, so no tile is skipped and
 * G_ij = (1/V - [j = y_i]) / n_valid on the non-ignored rows:
 *   dE = G c = 0 exactly,
 *   dC_j = sum_i G_ij e_i = (sum over valid i of e_i) / (V n_valid)
 *                           - (sum over valid i with y_i = j of e_i) / n_valid.
 * Sizes are ragged (N, V not multiples of the 256 tiles).  Exit status 0 on
 * success; the first failed check is printed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "cce.h"

#define N 300
#define D 64
#define V 1000
#define IGNORE (-100)

static int fails = 0;
#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      fprintf(stderr, "FAIL: " __VA_ARGS__);     \
      fprintf(stderr, "\n");                     \
      fails++;                                   \
    }                                            \
  } while (0)

#define HIP(x)                                                                 \
  do {                                                                         \
    hipError_t err_ = (x);                                                     \
    if (err_ != hipSuccess) {                                                  \
      fprintf(stderr, "HIP error %s at %s\n", hipGetErrorString(err_), #x);   \
      exit(2);                                                                 \
    }                                                                          \
  } while (0)

/* bf16 bits of a float that bf16 holds exactly (multiples of 1/8 below 2) */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

int main(void) {
  static uint16_t e_h[N * D], c_h[V * D];
  static int64_t t_h[N];
  static float ev[N][D];
  int n_valid = 0;
  for (int i = 0; i < N; ++i) {
    for (int d = 0; d < D; ++d) {
      ev[i][d] = (float)((i * 7 + d * 3) % 17 - 8) / 8.0f;
      e_h[i * D + d] = to_bf16(ev[i][d]);
    }
    t_h[i] = (i % 10 == 3) ? IGNORE : (int64_t)((i * 37) % V);
    n_valid += t_h[i] != IGNORE;
  }
  memset(c_h, 0, sizeof c_h);

  void *e, *c, *state, *ws;
  int64_t* t;
  float *loss, *lse, *dE, *dC;
  int32_t* nv;
  hipStream_t st;
  HIP(hipStreamCreate(&st));
  const size_t state_bytes = cce_state_size(N, D, V, CCE_DTYPE_BF16);
  const size_t ws_bytes = cce_workspace_size(N, D, V, CCE_DTYPE_BF16, 0);
  CHECK(state_bytes > 0 && ws_bytes > 0, "state and workspace sizes");
  HIP(hipMalloc(&e, sizeof e_h));
  HIP(hipMalloc(&c, sizeof c_h));
  HIP(hipMalloc((void**)&t, sizeof t_h));
  HIP(hipMalloc((void**)&loss, 4));
  HIP(hipMalloc((void**)&lse, N * 4));
  HIP(hipMalloc((void**)&nv, 4));
  HIP(hipMalloc((void**)&dE, N * D * 4));
  HIP(hipMalloc((void**)&dC, V * D * 4));
  HIP(hipMalloc(&state, state_bytes));
  HIP(hipMalloc(&ws, ws_bytes));
  HIP(hipMemcpy(e, e_h, sizeof e_h, hipMemcpyHostToDevice));
  HIP(hipMemcpy(c, c_h, sizeof c_h, hipMemcpyHostToDevice));
  HIP(hipMemcpy(t, t_h, sizeof t_h, hipMemcpyHostToDevice));

  /* argument faults come back before any launch */
  CHECK(cce_forward(NULL, c, NULL, t, N, D, V, CCE_DTYPE_BF16, IGNORE, CCE_REDUCTION_MEAN, 0.f, 0.f, 0.f, loss,
                    lse, nv, state, state_bytes, (cce_stream_t)st) == CCE_ERR_INVALID_ARG,
        "null e must be CCE_ERR_INVALID_ARG");
  CHECK(cce_forward(e, c, NULL, t, N, D, V, CCE_DTYPE_BF16, IGNORE, CCE_REDUCTION_MEAN, 0.f, 0.f, 0.f, loss, lse,
                    nv, state, 1024, (cce_stream_t)st) == CCE_ERR_WORKSPACE,
        "a short state must be CCE_ERR_WORKSPACE");
  CHECK(strlen(cce_status_string(CCE_ERR_WORKSPACE)) > 0, "status string");

  int s = cce_forward(e, c, NULL, t, N, D, V, CCE_DTYPE_BF16, IGNORE, CCE_REDUCTION_MEAN, 0.f, 0.f, 0.f, loss, lse,
                      nv, state, state_bytes, (cce_stream_t)st);
  CHECK(s == CCE_OK, "forward: %s", cce_status_string(s));
  const float one = 1.0f;
  float* g;
  HIP(hipMalloc((void**)&g, 4));
  HIP(hipMemcpy(g, &one, 4, hipMemcpyHostToDevice));
  s = cce_backward(e, c, NULL, t, N, D, V, CCE_DTYPE_BF16, IGNORE, CCE_REDUCTION_MEAN, 0.f, 0.f, 0.f, lse, g,
                   1 /* filter */, CCE_ACCUM_DETERMINISTIC, 0, CCE_GRAD_FLOAT32, dE, dC, NULL, state, state_bytes,
                   ws, ws_bytes, (cce_stream_t)st);
  CHECK(s == CCE_OK, "backward: %s", cce_status_string(s));
  cce_stats stats;
  s = cce_read_stats(state, state_bytes, N, V, (cce_stream_t)st, &stats);
  CHECK(s == CCE_OK, "read_stats: %s", cce_status_string(s));

  static float lse_o[N], dE_o[N * D], dC_o[V * D];
  float loss_o;
  int32_t nv_o;
  HIP(hipMemcpy(&loss_o, loss, 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(&nv_o, nv, 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(lse_o, lse, sizeof lse_o, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(dE_o, dE, sizeof dE_o, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(dC_o, dC, sizeof dC_o, hipMemcpyDeviceToHost));

  const double lnV = log((double)V);
  CHECK(nv_o == n_valid, "n_valid %d, expected %d", nv_o, n_valid);
  CHECK(stats.n_valid == n_valid && stats.bad_targets == 0, "stats n_valid / bad_targets");
  CHECK(stats.tiles_kept == stats.tiles_total, "uniform softmax: no tile skipped (%lld of %lld kept)",
        (long long)stats.tiles_kept, (long long)stats.tiles_total);
  CHECK(fabs(loss_o - lnV) <= 1e-3 * lnV, "mean loss %.7f, expected ln V = %.7f", loss_o, lnV);
  double worst = 0;
  for (int i = 0; i < N; ++i) worst = fmax(worst, fabs(lse_o[i] - lnV));
  CHECK(worst <= 2e-3, "LSE off ln V by %g", worst);
  int nz = 0;
  for (int k = 0; k < N * D; ++k) nz += dE_o[k] != 0.0f;
  CHECK(nz == 0, "dE must be exactly 0 with c = 0 (%d nonzero)", nz);
  /* dC closed form, in double */
  static double ref[V][D];
  double sum_e[D] = {0};
  for (int i = 0; i < N; ++i)
    if (t_h[i] != IGNORE)
      for (int d = 0; d < D; ++d) sum_e[d] += ev[i][d];
  for (int j = 0; j < V; ++j)
    for (int d = 0; d < D; ++d) ref[j][d] = sum_e[d] / ((double)V * n_valid);
  for (int i = 0; i < N; ++i)
    if (t_h[i] != IGNORE)
      for (int d = 0; d < D; ++d) ref[t_h[i]][d] -= ev[i][d] / n_valid;
  double num = 0, den = 0;
  for (int j = 0; j < V; ++j)
    for (int d = 0; d < D; ++d) {
      const double x = dC_o[j * D + d] - ref[j][d];
      num += x * x;
      den += ref[j][d] * ref[j][d];
    }
  const double rel = sqrt(num / den);
  CHECK(rel <= 5e-3, "dC relative Frobenius error %g", rel);

  hipFree(e); hipFree(c); hipFree(t); hipFree(loss); hipFree(lse); hipFree(nv);
  hipFree(dE); hipFree(dC); hipFree(state); hipFree(ws); hipFree(g);
  hipStreamDestroy(st);
  if (fails) return 1;
  printf("cce C ABI check ok: loss %.6f (ln V %.6f), n_valid %d, dC rel err %.2e, %lld/%lld tiles\n", loss_o, lnV,
         nv_o, rel, (long long)stats.tiles_kept, (long long)stats.tiles_total);
  return 0;
}
