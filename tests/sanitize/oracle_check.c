/* The fp64 C oracle (oracle/gla_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: forward, backward and decode on small seeded
 * inputs, dense and packed (with an empty sequence), with and without S0 and
 * dS_T, with a reset gate; results checked finite. Exit status 0 when clean. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gla_oracle_fwd(const float *q, const float *k, const float *v, const float *lg,
                   const float *S0, const int64_t *cu, int B, int T, int H, int dk, int dv, int N,
                   double *o, double *ST, int nthreads);
int gla_oracle_bwd(const float *q, const float *k, const float *v, const float *lg,
                   const float *dO, const float *S0, const float *dST, const int64_t *cu, int B,
                   int T, int H, int dk, int dv, int N, double *dq, double *dkk, double *dvv,
                   double *dl, double *dS0, int nthreads);
int gla_oracle_decode(const float *q, const float *k, const float *v, const float *lg, double *S,
                      double *o, int N, int H, int dk, int dv, int nthreads);

static unsigned s = 12345u;
static float rnd(void) {
  s = s * 1664525u + 1013904223u;
  return (float)((s >> 8) & 0xffff) / 65536.0f - 0.5f;
}
static float *fill(size_t n) {
  float *p = (float *)malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = rnd();
  return p;
}
static int all_finite(const double *p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

int main(void) {
  int bad = 0;
  for (int packed = 0; packed < 2; ++packed) {
    const int H = 2, dk = 8, dv = 6, T = 37;
    const int B = packed ? 1 : 2, N = packed ? 4 : 2;
    const int64_t cu[5] = {0, 0, 10, 11, 37};
    const size_t tok = (size_t)B * T * H;
    float *q = fill(tok * dk), *k = fill(tok * dk), *v = fill(tok * dv), *dO = fill(tok * dv);
    float *lg = fill(tok);
    for (size_t i = 0; i < tok; ++i) lg[i] = -0.1f + 0.05f * lg[i];
    lg[3 * H] = -INFINITY; /* a reset */
    float *S0 = fill((size_t)N * H * dk * dv), *dST = fill((size_t)N * H * dk * dv);
    double *o = calloc(tok * dv, sizeof(double)), *ST = calloc((size_t)N * H * dk * dv, sizeof(double));
    double *dq = calloc(tok * dk, sizeof(double)), *dkk = calloc(tok * dk, sizeof(double));
    double *dvv = calloc(tok * dv, sizeof(double)), *dl = calloc(tok, sizeof(double));
    double *dS0 = calloc((size_t)N * H * dk * dv, sizeof(double));
    const int64_t *c = packed ? cu : NULL;
    for (int with = 0; with < 2; ++with) {
      gla_oracle_fwd(q, k, v, lg, with ? S0 : NULL, c, B, T, H, dk, dv, N, o, ST, 2);
      bad |= !all_finite(o, tok * dv) || !all_finite(ST, (size_t)N * H * dk * dv);
      if (gla_oracle_bwd(q, k, v, lg, dO, with ? S0 : NULL, with ? dST : NULL, c, B, T, H, dk, dv,
                         N, dq, dkk, dvv, dl, dS0, 2) < 0)
        bad = 1;
      bad |= !all_finite(dq, tok * dk) || !all_finite(dl, tok) || !all_finite(dS0, (size_t)N * H * dk * dv);
    }
    double *S = calloc((size_t)N * H * dk * dv, sizeof(double)), *od = calloc((size_t)N * H * dv, sizeof(double));
    gla_oracle_decode(q, k, v, lg, S, od, N, H, dk, dv, 2);
    bad |= !all_finite(od, (size_t)N * H * dv);
    free(q); free(k); free(v); free(dO); free(lg); free(S0); free(dST); free(o); free(ST);
    free(dq); free(dkk); free(dvv); free(dl); free(dS0); free(S); free(od);
  }
  printf("oracle_check: %s\n", bad ? "FAILED" : "ok");
  return bad;
}
