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
// This path serves fp32 callers that need fp32 accuracy. One 256-thread
// workgroup owns one work item (a run of tokens of one sequence) for one head
// and a slice of DVS = 32 state columns; the state slice lives in LDS, Q and K
// are staged 32 key-dimensions at a time. The four contractions (scores Q K^T,
// the state read Q S, P V and the state update K^T V) run on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulation), each
// wavefront owning whole 16 x 16 output tiles.
#include "bf16_blocks.h"
#include "gla_common.h"
#include "gla_internal.h"

namespace gla {

constexpr int kF32Slice = 32;  // state columns per workgroup
constexpr int kF32DkBlk = 32;  // key dimensions staged at a time

// D += A B for a 16 x 4 A and a 4 x 16 B, fp32. Lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16]; it holds D[4 (l / 16) + r][l % 16] in element r.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

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
template <int C, int DK, typename Tout, bool STATE_PASS, bool REV = false, typename Tin = float>
__global__ __launch_bounds__(256) void chunk_f32_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ lg, const float *__restrict__ S0, float *__restrict__ ST,
    Tout *__restrict__ o, const WorkItem *__restrict__ items, const int *__restrict__ n_items,
    float *__restrict__ slots, float *__restrict__ slot_gamma, int T, int H, int gts, int DV) {
  constexpr int DVS = kF32Slice, KB = kF32DkBlk;
  constexpr int NT = C / 16;               // 16-row tiles of a chunk
  constexpr int NST = NT * (NT + 1) / 2;   // lower-triangular score tiles
  constexpr int SPW = (NST + 3) / 4;       // score tiles per wavefront (at most)
  constexpr int NCT = DVS / 16;            // 16-column tiles of the slice
  constexpr int OPW = NT * NCT / 4;        // output tiles per wavefront
  constexpr int UPW = (KB / 16) * NCT / 4; // state tiles per wavefront per key block
  static_assert(NT * NCT % 4 == 0 && (KB / 16) * NCT % 4 == 0 && KB % 16 == 0, "tiling");
  static_assert(C == 64 || C == 128, "the gate scan covers one or two wavefronts");

  __shared__ float Qb[C][KB + 1];
  __shared__ float Kb[C][KB + 1];
  __shared__ float Vs[C][DVS + 1];
  __shared__ float P[C][C + 1];
  __shared__ float Ss[DK][DVS + 1];
  __shared__ float bcum[C], lam[C], kap[C];
  __shared__ int rpos[C];  // last reset at or before position i (-1: none)
  __shared__ float gam_s, gsum_s;

  const int n_slices = DV / DVS;
  const int slice = blockIdx.x % n_slices;
  const int h = (blockIdx.x / n_slices) % H;
  const int it = blockIdx.x / (n_slices * H);
  if (items && it >= *n_items) return;
  const WorkItem w = item_for(items, it, T);
  const int c0 = slice * DVS;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), ln = tid % 16, l4 = (tid / 16) % 4;
  const size_t dkdv = (size_t)DK * DV;
  const int sb = w.seq_begin, se = w.seq_end;
  auto mrow = [&](int t) -> size_t { return (size_t)(REV ? sb + se - 1 - t : t); };
  // Key blocks of a chunk go through registers: the block after the one being
  // computed is loaded while the matrix cores work on LDS (thread tid moves
  // elements tid + 256 e, e < EPT, of the block's C x KB tile).
  constexpr int EPT = C * KB / 256;
  auto load_blk = [&](const Tin *src, int t0, int n, int db, float (&x)[EPT]) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = (tid + 256 * e) / KB, dd = (tid + 256 * e) % KB;
      x[e] = i < n ? load_as_f32(src, (mrow(t0 + i) * H + h) * DK + db + dd) : 0.f;
    }
  };
  // the chunk's log-gate (thread tid < C holds token tid) and V slice elements
  // (tid + 256 e, e < VPT, of the C x DVS tile), also loaded a chunk ahead
  constexpr int VPT = C * DVS / 256;
  auto load_gate = [&](int t0, int n) -> float {
    if (tid >= n) return 0.f;
    if (REV) {
      const int u = t0 + tid - sb;
      return u == 0 ? 0.f : lg[(size_t)(se - u) * gts + h];
    }
    return lg[(size_t)(t0 + tid) * gts + h];
  };
  auto load_v = [&](int t0, int n, float (&x)[VPT]) {
#pragma unroll
    for (int e = 0; e < VPT; ++e) {
      const int j = (tid + 256 * e) / DVS, c = (tid + 256 * e) % DVS;
      x[e] = j < n ? load_as_f32(v, (mrow(t0 + j) * H + h) * DV + c0 + c) : 0.f;
    }
  };
  auto store_blk = [&](float (&dst)[C][KB + 1], const float (&x)[EPT], const float *scale) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = (tid + 256 * e) / KB, dd = (tid + 256 * e) % KB;
      dst[i][dd] = scale ? x[e] * scale[i] : x[e];
    }
  };

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

  // registers of the next loads: gate and V of the chunk, Q and K blocks of the
  // scores, K blocks of the state update. At chunk 64 a chunk's first loads are
  // issued during the previous chunk's last state-update block; at chunk 128
  // (twice the registers per load) at the chunk's start.
  constexpr bool kAhead = C == 64;
  float gx = 0.f, vx[VPT], qx[EPT], kx[EPT], ka[EPT];
  auto first_loads = [&](int t1) {
    const int n1 = min(C, w.tok_end - t1);
    gx = load_gate(t1, n1);
    load_v(t1, n1, vx);
    if (STATE_PASS) {
      load_blk(k, t1, n1, 0, ka);
    } else {
      load_blk(q, t1, n1, 0, qx);
      load_blk(k, t1, n1, 0, kx);
    }
  };
  if (kAhead && w.tok_begin < w.tok_end) first_loads(w.tok_begin);

  for (int t0 = w.tok_begin; t0 < w.tok_end; t0 += C) {
    const int n = min(C, w.tok_end - t0);
    if (!kAhead) first_loads(t0);
    __syncthreads();
    // gates: inclusive scan of the chunk's log-gates (padding rows add 0), one
    // wavefront scan per 64 tokens; a second 64 adds the first one's total.
    // A reset gate adds 0 and cuts every product of gates that spans it: the
    // chunk decay, e^{b_i} from the chunk's first reset on, kappa_j before its
    // last reset, and score keys before the query's last reset.
    if (tid < C) {
      const bool rst = is_reset(gx);
      const int ri = last_set_upto(__builtin_amdgcn_ballot_w64(rst), tid % 64);
      bcum[tid] = wave_inclusive_scan(rst ? 0.f : gx);
      rpos[tid] = ri < 0 ? -1 : (tid & ~63) + ri;
    }
#pragma unroll
    for (int e = 0; e < VPT; ++e) Vs[(tid + 256 * e) / DVS][(tid + 256 * e) % DVS] = vx[e];
    __syncthreads();
    if constexpr (C == 128) {
      const float first = bcum[63];
      const int r_first = rpos[63];
      __syncthreads();
      if (tid >= 64 && tid < 128) {
        bcum[tid] += first;
        if (rpos[tid] < 0) rpos[tid] = r_first;
      }
      __syncthreads();
    }
    const float blast = bcum[n - 1];
    const int rlast = rpos[n - 1];
    if (tid < C) {
      lam[tid] = rpos[tid] < 0 ? expf(bcum[tid]) : 0.f;
      kap[tid] = tid < rlast ? 0.f : expf(blast - bcum[tid]);
    }
    if (tid == 0) gam_s = rlast < 0 ? expf(blast) : 0.f;
    gsum += rlast < 0 ? blast : -__builtin_huge_valf();

    if (!STATE_PASS) {
      // score tiles t = wave, wave + 4, ... (lower triangle, row-major) and the
      // output tiles u -> (row tile, column tile), accumulated over key blocks
      f32x4 sacc[SPW], oacc[OPW];
#pragma unroll
      for (int s = 0; s < SPW; ++s) sacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < OPW; ++u) oacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int db = 0; db < DK; db += KB) {
        __syncthreads();
        store_blk(Qb, qx, nullptr);
        store_blk(Kb, kx, nullptr);
        __syncthreads();
        if (db + KB < DK) {
          load_blk(q, t0, n, db + KB, qx);
          load_blk(k, t0, n, db + KB, kx);
        } else if (kAhead) {  // the state update's first block, in flight through P V
          load_blk(k, t0, n, 0, ka);
        }
        // scores Q K^T: A = Q rows, B = K^T
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
          const int t = wave + 4 * s;
          if (t < NST) {
            const int ti = tile_ti(t), tj = tile_tj(t);
#pragma unroll
            for (int ks = 0; ks < KB / 4; ++ks)
              sacc[s] = mfma_f32(Qb[16 * ti + ln][4 * ks + l4], Kb[16 * tj + ln][4 * ks + l4], sacc[s]);
          }
        }
        // state read Q S over this key block
#pragma unroll
        for (int u = 0; u < OPW; ++u) {
          const int ot = wave + 4 * u, ti = ot / NCT, tc = ot % NCT;
#pragma unroll
          for (int ks = 0; ks < KB / 4; ++ks)
            oacc[u] = mfma_f32(Qb[16 * ti + ln][4 * ks + l4], Ss[db + 4 * ks + l4][16 * tc + ln], oacc[u]);
        }
      }
      // decay mask: P[i][j] = score * e^{b_i - b_j} for j <= i with no reset in
    // (j, i], else 0
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
        const int t = wave + 4 * s;
        if (t < NST) {
          const int ti = tile_ti(t), tj = tile_tj(t), j = 16 * tj + ln;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * ti + 4 * l4 + r;
            P[i][j] = (j <= i && j >= rpos[i]) ? sacc[s][r] * expf(bcum[i] - bcum[j]) : 0.f;
          }
        }
      }
      __syncthreads();
      // o = e^{b_i} (Q S) + P V, keys up to the end of the row tile
#pragma unroll
      for (int u = 0; u < OPW; ++u) {
        const int ot = wave + 4 * u, ti = ot / NCT, tc = ot % NCT;
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[u][r] *= lam[16 * ti + 4 * l4 + r];
        for (int ks = 0; ks < 4 * (ti + 1); ++ks)
          oacc[u] = mfma_f32(P[16 * ti + ln][4 * ks + l4], Vs[4 * ks + l4][16 * tc + ln], oacc[u]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ti + 4 * l4 + r;
          if (i < n) store_from_f32(o, (mrow(t0 + i) * H + h) * DV + c0 + 16 * tc + ln, oacc[u][r]);
        }
      }
    }
    // state advance: S <- gamma S + (kappa K)^T V, one key block at a time;
    // each wavefront owns whole 16 x 16 tiles of the block's state rows
    if (!kAhead && !STATE_PASS) load_blk(k, t0, n, 0, ka);
    for (int db = 0; db < DK; db += KB) {
      __syncthreads();
      store_blk(Kb, ka, kap);
      __syncthreads();
      if (db + KB < DK) {
        load_blk(k, t0, n, db + KB, ka);
      } else if (kAhead && t0 + C < w.tok_end) {  // the next chunk's first loads
        first_loads(t0 + C);
      }
      const float gam = gam_s;
#pragma unroll
      for (int u = 0; u < UPW; ++u) {
        const int ut = wave + 4 * u, td = ut / NCT, tc = ut % NCT;
        f32x4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = gam * Ss[db + 16 * td + 4 * l4 + r][16 * tc + ln];
#pragma unroll
        for (int ks = 0; ks < C / 4; ++ks)
          acc = mfma_f32(Kb[4 * ks + l4][16 * td + ln], Vs[4 * ks + l4][16 * tc + ln], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) Ss[db + 16 * td + 4 * l4 + r][16 * tc + ln] = acc[r];
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

template <int C, int DK, typename Tin, typename Tout, bool SP, bool REV = false>
static hipError_t launch_f32_t(const Tin *q, const Tin *k, const Tin *v, const float *g,
                               const float *S0, float *S_T, void *o, const FwdDims &d,
                               const WorkItem *items, const int *n_items, int grid_items,
                               float *slots, float *slot_gamma, hipStream_t stream) {
  const long blocks = (long)grid_items * d.H * (d.dv / kF32Slice);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_f32_kernel<C, DK, Tout, SP, REV, Tin>), dim3(blocks), dim3(256), 0,
                     stream, q, k, v, g, S0, S_T, static_cast<Tout *>(o), items, n_items, slots,
                     slot_gamma, d.T, d.H, d.gts, d.dv);
  return hipGetLastError();
}

// fp32 inputs: the fp32 forward (d_k in {64, 96, 128}, bf16 or fp32 o) and the
// backward's runs (fp32 o; time-reversed or not; d_k 192 for the 96 x 192
// heads' dq and dk runs).
template <int C, int DK>
static hipError_t launch_f32_c(const float *q, const float *k, const float *v, const float *g,
                               const float *S0, float *S_T, void *o, bool out_bf16,
                               const FwdDims &d, const WorkItem *items, const int *n_items,
                               int grid_items, float *slots, float *slot_gamma, bool state_pass,
                               hipStream_t stream) {
  if (d.rev) {  // time-reversed runs of the backward: fp32 outputs
    if (out_bf16) return hipErrorInvalidValue;
    if (state_pass)
      return launch_f32_t<C, DK, float, float, true, true>(q, k, v, g, S0, S_T, o, d, items,
                                                           n_items, grid_items, slots, slot_gamma,
                                                           stream);
    return launch_f32_t<C, DK, float, float, false, true>(q, k, v, g, S0, S_T, o, d, items,
                                                          n_items, grid_items, slots, slot_gamma,
                                                          stream);
  }
  if (state_pass)
    return launch_f32_t<C, DK, float, float, true>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                                   grid_items, slots, slot_gamma, stream);
  if constexpr (DK != 192) {
    if (out_bf16)
      return launch_f32_t<C, DK, float, uint16_t, false>(q, k, v, g, S0, S_T, o, d, items,
                                                         n_items, grid_items, slots, slot_gamma,
                                                         stream);
  } else {
    if (out_bf16) return hipErrorInvalidValue;
  }
  return launch_f32_t<C, DK, float, float, false>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                                  grid_items, slots, slot_gamma, stream);
}

// bf16 inputs through the fp32 kernel: the backward's runs for the 96 x 192
// heads (d_k 96 or 192, fp32 o), which the bf16 kernels do not cover.
template <int C, int DK>
static hipError_t launch_f32_bf16in(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                    const float *g, const float *S0, float *S_T, void *o,
                                    bool out_bf16, const FwdDims &d, const WorkItem *items,
                                    const int *n_items, int grid_items, float *slots,
                                    float *slot_gamma, bool state_pass, hipStream_t stream) {
  if (out_bf16) return hipErrorInvalidValue;
  if (d.rev) {
    if (state_pass)
      return launch_f32_t<C, DK, uint16_t, float, true, true>(q, k, v, g, S0, S_T, o, d, items,
                                                              n_items, grid_items, slots,
                                                              slot_gamma, stream);
    return launch_f32_t<C, DK, uint16_t, float, false, true>(q, k, v, g, S0, S_T, o, d, items,
                                                             n_items, grid_items, slots,
                                                             slot_gamma, stream);
  }
  if (state_pass)
    return launch_f32_t<C, DK, uint16_t, float, true>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                                      grid_items, slots, slot_gamma, stream);
  return launch_f32_t<C, DK, uint16_t, float, false>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                                     grid_items, slots, slot_gamma, stream);
}

hipError_t launch_chunk_f32(const void *q, const void *k, const void *v, const float *g,
                            const float *S0, float *S_T, void *o, bool in_bf16, bool out_bf16,
                            const FwdDims &d, const WorkItem *items, const int *n_items,
                            int grid_items, float *slots, float *slot_gamma, bool state_pass,
                            hipStream_t stream) {
  if (d.hg != 1) return hipErrorInvalidValue;  // head groups: the bf16 kernel only
  if (d.dot_x) return hipErrorInvalidValue;  // row dots: bf16 chunk-64 kernel only
  if (in_bf16) {
    const auto *qb = static_cast<const uint16_t *>(q), *kb = static_cast<const uint16_t *>(k),
               *vb = static_cast<const uint16_t *>(v);
    if (d.dk == 96)
      return d.C == 64 ? launch_f32_bf16in<64, 96>(qb, kb, vb, g, S0, S_T, o, out_bf16, d, items,
                                                   n_items, grid_items, slots, slot_gamma,
                                                   state_pass, stream)
                       : launch_f32_bf16in<128, 96>(qb, kb, vb, g, S0, S_T, o, out_bf16, d,
                                                    items, n_items, grid_items, slots,
                                                    slot_gamma, state_pass, stream);
    if (d.dk == 192)
      return d.C == 64 ? launch_f32_bf16in<64, 192>(qb, kb, vb, g, S0, S_T, o, out_bf16, d,
                                                    items, n_items, grid_items, slots,
                                                    slot_gamma, state_pass, stream)
                       : launch_f32_bf16in<128, 192>(qb, kb, vb, g, S0, S_T, o, out_bf16, d,
                                                     items, n_items, grid_items, slots,
                                                     slot_gamma, state_pass, stream);
    return hipErrorInvalidValue;
  }
  const auto *qf = static_cast<const float *>(q), *kf = static_cast<const float *>(k),
             *vf = static_cast<const float *>(v);
#define GLA_F32_CASE(CC, DD)                                                                   \
  if (d.C == CC && d.dk == DD)                                                                \
    return launch_f32_c<CC, DD>(qf, kf, vf, g, S0, S_T, o, out_bf16, d, items, n_items,       \
                                grid_items, slots, slot_gamma, state_pass, stream);
  GLA_F32_CASE(64, 64)
  GLA_F32_CASE(64, 96)
  GLA_F32_CASE(64, 128)
  GLA_F32_CASE(64, 192)
  GLA_F32_CASE(128, 64)
  GLA_F32_CASE(128, 96)
  GLA_F32_CASE(128, 128)
  GLA_F32_CASE(128, 192)
#undef GLA_F32_CASE
  return hipErrorInvalidValue;
}

}  // namespace gla
