// Chunked GLA forward for fp32 inputs, in fp32 vector arithmetic.
//
// Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), "Challenge 1":
// within a chunk the output is decay-masked linear attention over the chunk
// plus the query's read of the running state, and the state then advances by
// the decay compounded over the chunk. With b_i the in-chunk inclusive
// cumulative log-gate (i = 0 .. n-1 over the chunk's n tokens):
//
//   O = diag(e^{b}) Q S + ((Q K^T) .* D) V,   D_ij = e^{b_i - b_j} (j <= i)
//   S <- e^{b_{n-1}} S + (diag(e^{b_{n-1} - b}) K)^T V
//
// D is evaluated per element as the exponential of a difference (never as a
// product e^{b_i} e^{-b_j}, which overflows for strong decay).
//
// This path serves fp32 callers that need fp32 accuracy; the bf16 path runs
// the same algebra on the matrix cores. One 256-thread workgroup owns one
// work item (a run of tokens of one sequence) for one head and a slice of
// DVS = 32 state columns; the state slice lives in LDS, Q and K are staged
// 32 key-dimensions at a time.
#include "gla_common.h"
#include "gla_internal.h"

namespace gla {

constexpr int kF32Slice = 32;  // state columns per workgroup
constexpr int kF32DkBlk = 32;  // key dimensions staged at a time

__device__ __forceinline__ WorkItem item_for(const WorkItem *items, int it, int T) {
  if (items) return items[it];
  WorkItem w;
  w.tok_begin = it * T;
  w.tok_end = (it + 1) * T;
  w.seq = it;
  w.state_in = -1;
  w.state_out = -1;
  w.seq_begin = w.tok_begin;
  w.seq_end = w.tok_end;
  w.pad = 0;
  return w;
}

// REV: the time-reversed run of the backward: logical token t of a sequence
// [sb, se) reads and writes memory row sb + se - 1 - t, and its gate is the
// log-gate of row se - (t - sb) (0 for t = sb).
template <int C, int DK, typename Tout, bool STATE_PASS, bool REV = false>
__global__ __launch_bounds__(256) void chunk_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ lg, const float *__restrict__ S0, float *__restrict__ ST,
    Tout *__restrict__ o, const WorkItem *__restrict__ items, const int *__restrict__ n_items,
    float *__restrict__ slots, float *__restrict__ slot_gamma, int T, int H, int gts, int DV) {
  constexpr int DVS = kF32Slice, KB = kF32DkBlk;
  constexpr int NPE = C * C / 256;    // score entries per thread
  constexpr int NOE = C * DVS / 256;  // output entries per thread
  constexpr int NSE = KB * DVS / 256; // state entries per thread per key block
  static_assert(NPE >= 1 && NOE >= 1 && NSE >= 1, "tile too small");

  __shared__ float Qb[C][KB + 1];
  __shared__ float Kb[C][KB + 1];
  __shared__ float Vs[C][DVS + 1];
  __shared__ float P[C][C + 1];
  __shared__ float Ss[DK][DVS];
  __shared__ float bcum[C], lam[C], kap[C];
  __shared__ float gam_s, gsum_s;

  const int n_slices = DV / DVS;
  const int slice = blockIdx.x % n_slices;
  const int h = (blockIdx.x / n_slices) % H;
  const int it = blockIdx.x / (n_slices * H);
  if (items && it >= *n_items) return;
  const WorkItem w = item_for(items, it, T);
  const int c0 = slice * DVS;
  const int tid = threadIdx.x;
  const size_t dkdv = (size_t)DK * DV;
  const int sb = w.seq_begin, se = w.seq_end;
  auto mrow = [&](int t) -> size_t { return (size_t)(REV ? sb + se - 1 - t : t); };

  // initial state slice
  const float *sin = nullptr;
  if (!STATE_PASS) {
    if (w.state_in >= 0) sin = slots + ((size_t)w.state_in * H + h) * dkdv;
    else if (S0) sin = S0 + ((size_t)w.seq * H + h) * dkdv;
  }
  for (int e = tid; e < DK * DVS; e += 256) {
    const int d = e / DVS, c = e % DVS;
    Ss[d][c] = sin ? sin[(size_t)d * DV + c0 + c] : 0.f;
  }
  float gsum = 0.f;  // total log-decay of the run (state pass)

  for (int t0 = w.tok_begin; t0 < w.tok_end; t0 += C) {
    const int n = min(C, w.tok_end - t0);
    __syncthreads();
    // gates: inclusive scan of the chunk's log-gates (padding rows add 0)
    if (tid < C) {
      float x = 0.f;
      if (tid < n) {
        if (REV) {
          const int u = t0 + tid - sb;
          x = u == 0 ? 0.f : lg[(size_t)(se - u) * gts + h];
        } else {
          x = lg[(size_t)(t0 + tid) * gts + h];
        }
      }
      bcum[tid] = x;
    }
    for (int e = tid; e < C * DVS; e += 256) {
      const int j = e / DVS, c = e % DVS;
      Vs[j][c] = (j < n) ? v[(mrow(t0 + j) * H + h) * DV + c0 + c] : 0.f;
    }
    for (int off = 1; off < C; off *= 2) {
      __syncthreads();
      float y = (tid < C && tid >= off) ? bcum[tid - off] : 0.f;
      __syncthreads();
      if (tid < C) bcum[tid] += y;
    }
    __syncthreads();
    const float blast = bcum[n - 1];
    if (tid < C) {
      lam[tid] = expf(bcum[tid]);
      kap[tid] = expf(blast - bcum[tid]);
    }
    if (tid == 0) gam_s = expf(blast);
    gsum += blast;

    float oacc[NOE];
    if (!STATE_PASS) {
      float pacc[NPE];
#pragma unroll
      for (int m = 0; m < NPE; ++m) pacc[m] = 0.f;
#pragma unroll
      for (int m = 0; m < NOE; ++m) oacc[m] = 0.f;
      // scores Q K^T and the state read Q S, one key block at a time
      for (int db = 0; db < DK; db += KB) {
        __syncthreads();
        for (int e = tid; e < C * KB; e += 256) {
          const int i = e / KB, dd = e % KB;
          const bool ok = i < n;
          Qb[i][dd] = ok ? q[(mrow(t0 + i) * H + h) * DK + db + dd] : 0.f;
          Kb[i][dd] = ok ? k[(mrow(t0 + i) * H + h) * DK + db + dd] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < NPE; ++m) {
          const int e = tid + 256 * m, i = e / C, j = e % C;
          float a = 0.f;
          if (j <= i) {
#pragma unroll 8
            for (int dd = 0; dd < KB; ++dd) a += Qb[i][dd] * Kb[j][dd];
          }
          pacc[m] += a;
        }
#pragma unroll
        for (int m = 0; m < NOE; ++m) {
          const int e = tid + 256 * m, i = e / DVS, c = e % DVS;
          float a = 0.f;
#pragma unroll 8
          for (int dd = 0; dd < KB; ++dd) a += Qb[i][dd] * Ss[db + dd][c];
          oacc[m] += a;
        }
      }
      // decay mask
#pragma unroll
      for (int m = 0; m < NPE; ++m) {
        const int e = tid + 256 * m, i = e / C, j = e % C;
        P[i][j] = (j <= i) ? pacc[m] * expf(bcum[i] - bcum[j]) : 0.f;
      }
      __syncthreads();
      // intra-chunk attention and the decayed state read
#pragma unroll
      for (int m = 0; m < NOE; ++m) {
        const int e = tid + 256 * m, i = e / DVS, c = e % DVS;
        float a = 0.f;
        for (int j = 0; j <= i; ++j) a += P[i][j] * Vs[j][c];
        const float r = lam[i] * oacc[m] + a;
        if (i < n) store_from_f32(o, (mrow(t0 + i) * H + h) * DV + c0 + c, r);
      }
    }
    // state advance: S <- gamma S + (kappa K)^T V, one key block at a time
    for (int db = 0; db < DK; db += KB) {
      __syncthreads();
      for (int e = tid; e < C * KB; e += 256) {
        const int j = e / KB, dd = e % KB;
        Kb[j][dd] = (j < n) ? k[(mrow(t0 + j) * H + h) * DK + db + dd] * kap[j] : 0.f;
      }
      __syncthreads();
      const float gam = gam_s;
#pragma unroll
      for (int m = 0; m < NSE; ++m) {
        const int e = tid + 256 * m, dd = e / DVS, c = e % DVS;
        float a = 0.f;
        for (int j = 0; j < C; ++j) a += Kb[j][dd] * Vs[j][c];
        Ss[db + dd][c] = gam * Ss[db + dd][c] + a;
      }
    }
  }
  __syncthreads();
  // final state of the run
  float *sout = nullptr;
  if (STATE_PASS) {
    sout = slots + ((size_t)w.state_out * H + h) * dkdv;
    if (slice == 0 && tid == 0) slot_gamma[(size_t)w.state_out * H + h] = gsum;
  } else if (w.state_out == -1 && ST) {
    sout = ST + ((size_t)w.seq * H + h) * dkdv;
  }
  if (sout) {
    for (int e = tid; e < DK * DVS; e += 256) {
      const int d = e / DVS, c = e % DVS;
      sout[(size_t)d * DV + c0 + c] = Ss[d][c];
    }
  }
}

template <int C, int DK, typename Tout, bool SP, bool REV = false>
static hipError_t launch_f32_t(const float *q, const float *k, const float *v, const float *g,
                               const float *S0, float *S_T, void *o, const FwdDims &d,
                               const WorkItem *items, const int *n_items, int grid_items,
                               float *slots, float *slot_gamma, hipStream_t stream) {
  const long blocks = (long)grid_items * d.H * (d.dv / kF32Slice);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_f32_kernel<C, DK, Tout, SP, REV>), dim3(blocks), dim3(256), 0, stream, q,
                     k, v, g, S0, S_T, static_cast<Tout *>(o), items, n_items, slots, slot_gamma,
                     d.T, d.H, d.gts, d.dv);
  return hipGetLastError();
}

template <int C, int DK>
static hipError_t launch_f32_c(const float *q, const float *k, const float *v, const float *g,
                               const float *S0, float *S_T, void *o, bool out_bf16,
                               const FwdDims &d, const WorkItem *items, const int *n_items,
                               int grid_items, float *slots, float *slot_gamma, bool state_pass,
                               hipStream_t stream) {
  if (d.rev) {  // time-reversed runs of the backward: fp32 outputs, d_k in {64, 128}
    if constexpr (DK == 96) {
      return hipErrorInvalidValue;
    } else {
      if (state_pass)
        return launch_f32_t<C, DK, float, true, true>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                                      grid_items, slots, slot_gamma, stream);
      if (out_bf16) return hipErrorInvalidValue;
      return launch_f32_t<C, DK, float, false, true>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                                     grid_items, slots, slot_gamma, stream);
    }
  }
  if (state_pass)
    return launch_f32_t<C, DK, float, true>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                            grid_items, slots, slot_gamma, stream);
  if (out_bf16)
    return launch_f32_t<C, DK, uint16_t, false>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                                grid_items, slots, slot_gamma, stream);
  return launch_f32_t<C, DK, float, false>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                           grid_items, slots, slot_gamma, stream);
}

hipError_t launch_chunk_f32(const float *q, const float *k, const float *v, const float *g,
                            const float *S0, float *S_T, void *o, bool out_bf16,
                            const FwdDims &d, const WorkItem *items, const int *n_items,
                            int grid_items, float *slots, float *slot_gamma, bool state_pass,
                            hipStream_t stream) {
  if (d.dot_x) return hipErrorInvalidValue;  // row dots: bf16 chunk-64 kernel only
  if (d.dk == 96) {
    if (d.C == 64)
      return launch_f32_c<64, 96>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                                  slots, slot_gamma, state_pass, stream);
    return launch_f32_c<128, 96>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                                 slots, slot_gamma, state_pass, stream);
  }
  if (d.C == 64) {
    if (d.dk == 128)
      return launch_f32_c<64, 128>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items,
                                   grid_items, slots, slot_gamma, state_pass, stream);
    return launch_f32_c<64, 64>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                                slots, slot_gamma, state_pass, stream);
  }
  if (d.dk == 128)
    return launch_f32_c<128, 128>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items,
                                  grid_items, slots, slot_gamma, state_pass, stream);
  return launch_f32_c<128, 64>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                               slots, slot_gamma, state_pass, stream);
}

}  // namespace gla
