/*
 * fp64 CPU oracle for the gated linear-attention (GLA) recurrence, in C.
 *
 * TEST INFRASTRUCTURE ONLY: linked by the tests and timed by the benchmark's
 * CPU-baseline leg; never by the HIP library. It shares no code with the GPU
 * path.
 *
 * Per (sequence, head), one token at a time, in fp64:
 *     S_t = exp(l_t) * S_{t-1} + k_t^T v_t,     o_t = q_t S_t
 * Source: Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), section
 * "GLA mixer" (decayed matrix state plus the rank-1 key/value outer product;
 * the readout queries the state), with the fixed per-head decay generalised
 * to a per-token log-gate l_t. Readout after the update; the gate scales only
 * the old state; varlen sequences restart from their own S0.
 *
 * The backward (gla_oracle_bwd) is the reverse-mode adjoint of the same
 * recurrence, walked back token by token from the stored forward states, as
 * the numpy oracle's recurrent_backward does (training differentiates through
 * every sequential state update: Laplace 3B on AWS Trainium2, "Challenge 3:
 * Backward-pass unrolling for a sequential recurrence").
 *
 * Inputs arrive as fp32 (bf16 inputs are passed as their exact fp32 values)
 * and are widened to double element by element, which is exact. OpenMP runs
 * independent (sequence, head) pairs in parallel; each pair is a plain serial
 * loop, so the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* q,k: [B,T,H,dk]; v: [B,T,H,dv]; lg: [B,T,H]; S0: [N,H,dk,dv] or NULL;
 * cu: [N+1] int64 or NULL (then N == B, each row of length T);
 * o: [B,T,H,dv] double; ST: [N,H,dk,dv] double or NULL.
 * Returns the number of threads used. */
int gla_oracle_fwd(const float *q, const float *k, const float *v, const float *lg,
                   const float *S0, const int64_t *cu, int B, int T, int H, int dk,
                   int dv, int N, double *o, double *ST, int nthreads) {
  int used = 1;
#ifdef _OPENMP
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
  const int nt = 1;
  (void)nthreads;
#endif
  const long pairs = (long)N * H;
#pragma omp parallel num_threads(nt)
  {
#ifdef _OPENMP
#pragma omp single
    used = omp_get_num_threads();
#endif
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
#pragma omp for schedule(dynamic, 1)
    for (long p = 0; p < pairs; ++p) {
      const int n = (int)(p / H), h = (int)(p % H);
      long row, start, end;
      if (cu) {
        row = 0;
        start = cu[n];
        end = cu[n + 1];
      } else {
        row = n;
        start = 0;
        end = T;
      }
      if (S0) {
        const float *s0 = S0 + ((size_t)n * H + h) * dk * dv;
        for (long i = 0; i < (long)dk * dv; ++i) S[i] = (double)s0[i];
      } else {
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
      }
      for (long t = start; t < end; ++t) {
        const size_t tok = ((size_t)row * T + t) * H + h;
        const double g = exp((double)lg[tok]);
        const float *kt = k + tok * dk, *vt = v + tok * dv, *qt = q + tok * dk;
        double *ot = o + tok * dv;
        for (int i = 0; i < dk; ++i) {
          const double ki = (double)kt[i];
          double *Si = S + (size_t)i * dv;
          for (int j = 0; j < dv; ++j) Si[j] = g * Si[j] + ki * (double)vt[j];
        }
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
          const double qi = (double)qt[i];
          const double *Si = S + (size_t)i * dv;
          for (int j = 0; j < dv; ++j) ot[j] += qi * Si[j];
        }
      }
      if (ST) memcpy(ST + ((size_t)n * H + h) * dk * dv, S, sizeof(double) * (size_t)dk * dv);
    }
    free(S);
  }
  return used;
}

/* One decode step: q,k: [N,H,dk]; v: [N,H,dv]; lg: [N,H]; S: [N,H,dk,dv]
 * double, updated in place; o: [N,H,dv] double. */
int gla_oracle_decode(const float *q, const float *k, const float *v, const float *lg,
                      double *S, double *o, int N, int H, int dk, int dv, int nthreads) {
  int used = 1;
#ifdef _OPENMP
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
  const int nt = 1;
  (void)nthreads;
#endif
  const long pairs = (long)N * H;
#pragma omp parallel num_threads(nt)
  {
#ifdef _OPENMP
#pragma omp single
    used = omp_get_num_threads();
#endif
#pragma omp for schedule(static)
    for (long p = 0; p < pairs; ++p) {
      const double g = exp((double)lg[p]);
      const float *kt = k + p * dk, *vt = v + p * dv, *qt = q + p * dk;
      double *Sp = S + (size_t)p * dk * dv, *op = o + (size_t)p * dv;
      for (int i = 0; i < dk; ++i) {
        double *Si = Sp + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) Si[j] = g * Si[j] + (double)kt[i] * (double)vt[j];
      }
      for (int j = 0; j < dv; ++j) op[j] = 0.0;
      for (int i = 0; i < dk; ++i) {
        const double *Si = Sp + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) op[j] += (double)qt[i] * Si[j];
      }
    }
  }
  return used;
}

/* Backward of gla_oracle_fwd for L = sum <dO, o> + sum <dS_T, S_T>.
 * q,k: [B,T,H,dk]; v, dO: [B,T,H,dv]; lg: [B,T,H]; S0, dST: [N,H,dk,dv] or
 * NULL (zeros); cu as in gla_oracle_fwd. Outputs (double): dq, dkk [B,T,H,dk],
 * dvv [B,T,H,dv], dl [B,T,H], dS0 [N,H,dk,dv]. With A = dL/dS_t, from the last
 * token back to the first:
 *     A += q_t^T dO_t                 (o_t = q_t S_t reads S_t)
 *     dq_t = S_t dO_t^T,  dk_t = A v_t^T,  dv_t = k_t A
 *     dl_t = g_t <A, S_{t-1}>         (S_t = g_t S_{t-1} + ..., g_t = exp(l_t))
 *     A = g_t A                       (now dL/dS_{t-1})
 * and dS0 = A after the first token. Every forward state of a sequence is
 * kept ((length + 1) d_k d_v doubles per thread). Returns the threads used,
 * or -1 if a state buffer could not be allocated. */
int gla_oracle_bwd(const float *q, const float *k, const float *v, const float *lg,
                   const float *dO, const float *S0, const float *dST, const int64_t *cu,
                   int B, int T, int H, int dk, int dv, int N, double *dq, double *dkk,
                   double *dvv, double *dl, double *dS0, int nthreads) {
  int used = 1, failed = 0;
#ifdef _OPENMP
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
  const int nt = 1;
  (void)nthreads;
#endif
  const long pairs = (long)N * H;
  const size_t mat = (size_t)dk * dv;
#pragma omp parallel num_threads(nt)
  {
#ifdef _OPENMP
#pragma omp single
    used = omp_get_num_threads();
#endif
    double *A = (double *)malloc(sizeof(double) * mat);
#pragma omp for schedule(dynamic, 1)
    for (long p = 0; p < pairs; ++p) {
      const int n = (int)(p / H), h = (int)(p % H);
      long row, start, end;
      if (cu) {
        row = 0;
        start = cu[n];
        end = cu[n + 1];
      } else {
        row = n;
        start = 0;
        end = T;
      }
      const long len = end > start ? end - start : 0;
      /* states[j] = S after j tokens of the sequence */
      double *states = (double *)malloc(sizeof(double) * mat * (size_t)(len + 1));
      if (!states || !A) {
#pragma omp atomic write
        failed = 1;
        free(states);
        continue;
      }
      if (S0) {
        const float *s0 = S0 + ((size_t)n * H + h) * mat;
        for (size_t i = 0; i < mat; ++i) states[i] = (double)s0[i];
      } else {
        memset(states, 0, sizeof(double) * mat);
      }
      for (long j = 0; j < len; ++j) {
        const size_t tok = ((size_t)row * T + start + j) * H + h;
        const double g = exp((double)lg[tok]);
        const float *kt = k + tok * dk, *vt = v + tok * dv;
        const double *Sp = states + (size_t)j * mat;
        double *Sn = states + (size_t)(j + 1) * mat;
        for (int i = 0; i < dk; ++i)
          for (int c = 0; c < dv; ++c)
            Sn[(size_t)i * dv + c] = g * Sp[(size_t)i * dv + c] + (double)kt[i] * (double)vt[c];
      }
      if (dST) {
        const float *d = dST + ((size_t)n * H + h) * mat;
        for (size_t i = 0; i < mat; ++i) A[i] = (double)d[i];
      } else {
        memset(A, 0, sizeof(double) * mat);
      }
      for (long j = len - 1; j >= 0; --j) {
        const size_t tok = ((size_t)row * T + start + j) * H + h;
        const double g = exp((double)lg[tok]);
        const float *qt = q + tok * dk, *kt = k + tok * dk, *vt = v + tok * dv;
        const float *dOt = dO + tok * dv;
        const double *Sj = states + (size_t)(j + 1) * mat; /* S_t */
        const double *Sm = states + (size_t)j * mat;       /* S_{t-1} */
        for (int i = 0; i < dk; ++i)
          for (int c = 0; c < dv; ++c) A[(size_t)i * dv + c] += (double)qt[i] * (double)dOt[c];
        double *dqt = dq + tok * dk, *dkt = dkk + tok * dk, *dvt = dvv + tok * dv;
        for (int i = 0; i < dk; ++i) {
          double sq = 0.0, sk = 0.0;
          for (int c = 0; c < dv; ++c) {
            sq += Sj[(size_t)i * dv + c] * (double)dOt[c];
            sk += A[(size_t)i * dv + c] * (double)vt[c];
          }
          dqt[i] = sq;
          dkt[i] = sk;
        }
        for (int c = 0; c < dv; ++c) {
          double sv = 0.0;
          for (int i = 0; i < dk; ++i) sv += (double)kt[i] * A[(size_t)i * dv + c];
          dvt[c] = sv;
        }
        double inner = 0.0;
        for (size_t i = 0; i < mat; ++i) inner += A[i] * Sm[i];
        dl[tok] = g * inner;
        for (size_t i = 0; i < mat; ++i) A[i] *= g;
      }
      memcpy(dS0 + ((size_t)n * H + h) * mat, A, sizeof(double) * mat);
      free(states);
    }
    free(A);
  }
  return failed ? -1 : used;
}
