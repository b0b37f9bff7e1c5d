// Chunked GLA forward for bf16 inputs on the CDNA4 matrix cores.
//
// Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), "Challenge 1":
// within each chunk the output is decay-masked linear attention over the
// chunk plus the query's read of the running state; chunks are independent
// except for the state, which advances by the decay compounded over the
// chunk. With b_i the in-chunk inclusive cumulative log-gate:
//
//   O = diag(e^{b}) (Q S) + ((Q K^T) .* D) V,     D_ij = e^{b_i - b_j}, j <= i
//   S <- e^{b_last} S + K^T (diag(e^{b_last - b}) V)
//
// Work decomposition (MI355X): one 256-thread workgroup (4 wavefronts) owns
// one work item (a run of one sequence's tokens) for one head and a 64-wide
// slice of the state's columns; it walks the item's chunks in order and keeps
// its d_k x 64 fp32 state slice in the matrix-core accumulator registers for
// the whole run. Wavefront w owns state and output columns 16w .. 16w+15.
// Per chunk:
//   1. the chunk's Q, K (row-major and transposed) and V (transposed) tiles
//      sit in LDS as bf16, with the in-chunk log2-domain gate prefix sums;
//   2. the lower-triangular 16x16 tiles of K Q^T are spread over the four
//      wavefronts (v_mfma_f32_16x16x32_bf16), masked by the decay
//      D_ij = 2^(b2_i - b2_j) evaluated per element, split into bf16 hi + lo
//      parts and written to LDS as P;
//   3. each wavefront computes Q S from its accumulator-resident state (the
//      accumulator layout is used directly as the B operand by permuting the
//      reduction order of Q to match), scales rows by e^{b_i}, adds P V, and
//      stores its 16 output columns;
//   4. it advances its state: S <- gamma S + K^T (kappa . V).
// Accuracy: bf16 inputs are exact operands; every value rounded on its way
// into an MFMA (P, S, kappa . V) is split into hi = bf16(x) and
// lo = bf16(x - hi) and both parts are multiplied, which keeps the products
// at ~16 significant bits with fp32 accumulation.
#include "gla_common.h"
#include "gla_internal.h"

namespace gla {

constexpr int kBfSlice = 64;  // state columns per workgroup (4 wavefronts x 16)

__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ WorkItem bf_item_for(const WorkItem *items, int it, int T) {
  if (items) return items[it];
  WorkItem w;
  w.tok_begin = it * T;
  w.tok_end = (it + 1) * T;
  w.seq = it;
  w.state_in = -1;
  w.state_out = -1;
  w.pad0 = w.pad1 = w.pad2 = 0;
  return w;
}

// bf16 element e (0..7) of a 16-byte vector
__device__ __forceinline__ uint32_t bf_elem(const u32x4 &x, int e) {
  const uint32_t w = x[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int C, int DK>
struct BfTile {
  static constexpr int PQ = DK + 8;  // row pitch (bf16) of Q and K: 4-bank row skew
  static constexpr int PT = C + 8;   // row pitch of K^T, V^T and P
  static constexpr int NKB = (C / 4) * (DK / 8);           // 4x8 blocks of a Q/K tile
  static constexpr int NVB = (C / 4) * (kBfSlice / 8);     // 4x8 blocks of the V slice
  static constexpr int KPT = (NKB + 255) / 256;            // blocks per thread
  static constexpr int VPT = (NVB + 255) / 256;
};

template <int C, int DK>
struct alignas(16) BfLds {
  using L = BfTile<C, DK>;
  uint16_t Q[C * L::PQ];
  uint16_t K[C * L::PQ];
  uint16_t Kt[DK * L::PT];
  uint16_t Vt[kBfSlice * L::PT];
  uint16_t Phi[C * L::PT];
  uint16_t Plo[C * L::PT];
  float b2[C];    // in-chunk inclusive prefix sum of the log-gates, in log2 units
  float lam[C];   // 2^(b2_i)
  float kap[C];   // 2^(b2_last - b2_j)
  float gam;      // 2^(b2_last): decay over the chunk
  float lsum;     // sum of the chunk's natural-log gates
};

template <int C, int DK, bool STATE_PASS>
struct BfPrefetch {
  using L = BfTile<C, DK>;
  u32x4 q[STATE_PASS ? 1 : L::KPT][4];
  u32x4 k[L::KPT][4];
  u32x4 v[L::VPT][4];
  float lg[C / 64];
};

template <int C, int DK, bool STATE_PASS>
__device__ __forceinline__ void bf_load(BfPrefetch<C, DK, STATE_PASS> &pf, const uint16_t *q,
                                        const uint16_t *k, const uint16_t *v, const float *lg,
                                        int t0, int n, int H, int h, int DV, int col0) {
  using L = BfTile<C, DK>;
  const int tid = threadIdx.x;
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int m = 0; m < L::KPT; ++m) {
    const int b = tid + 256 * m;
    const int jb = b / (DK / 8), db = b % (DK / 8);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 4 * jb + r;
      const bool ok = (b < L::NKB) && (j < n);
      const size_t off = ((size_t)(t0 + j) * H + h) * DK + 8 * db;
      pf.k[m][r] = ok ? *reinterpret_cast<const u32x4 *>(k + off) : z;
      if (!STATE_PASS) pf.q[m][r] = ok ? *reinterpret_cast<const u32x4 *>(q + off) : z;
    }
  }
#pragma unroll
  for (int m = 0; m < L::VPT; ++m) {
    const int b = tid + 256 * m;
    const int jb = b / (kBfSlice / 8), cb = b % (kBfSlice / 8);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 4 * jb + r;
      const bool ok = (b < L::NVB) && (j < n);
      pf.v[m][r] = ok ? *reinterpret_cast<const u32x4 *>(
                            v + ((size_t)(t0 + j) * H + h) * DV + col0 + 8 * cb)
                      : z;
    }
  }
  if (tid < 64) {
#pragma unroll
    for (int e = 0; e < C / 64; ++e) {
      const int j = tid * (C / 64) + e;
      pf.lg[e] = (j < n) ? lg[(size_t)(t0 + j) * H + h] : 0.f;
    }
  }
}

// Write a prefetched chunk into LDS: Q and K row-major, K and V transposed, and
// the gate prefix sums (wavefront 0).
template <int C, int DK, bool STATE_PASS>
__device__ __forceinline__ void bf_store(const BfPrefetch<C, DK, STATE_PASS> &pf,
                                         BfLds<C, DK> &s) {
  using L = BfTile<C, DK>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int m = 0; m < L::KPT; ++m) {
    const int b = tid + 256 * m;
    if (b < L::NKB) {
      const int jb = b / (DK / 8), db = b % (DK / 8);
      if (!STATE_PASS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          *reinterpret_cast<u32x4 *>(&s.Q[(4 * jb + r) * L::PQ + 8 * db]) = pf.q[m][r];
          *reinterpret_cast<u32x4 *>(&s.K[(4 * jb + r) * L::PQ + 8 * db]) = pf.k[m][r];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u32x2 w;
        w.x = bf_elem(pf.k[m][0], e) | (bf_elem(pf.k[m][1], e) << 16);
        w.y = bf_elem(pf.k[m][2], e) | (bf_elem(pf.k[m][3], e) << 16);
        *reinterpret_cast<u32x2 *>(&s.Kt[(8 * db + e) * L::PT + 4 * jb]) = w;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < L::VPT; ++m) {
    const int b = tid + 256 * m;
    if (b < L::NVB) {
      const int jb = b / (kBfSlice / 8), cb = b % (kBfSlice / 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u32x2 w;
        w.x = bf_elem(pf.v[m][0], e) | (bf_elem(pf.v[m][1], e) << 16);
        w.y = bf_elem(pf.v[m][2], e) | (bf_elem(pf.v[m][3], e) << 16);
        *reinterpret_cast<u32x2 *>(&s.Vt[(8 * cb + e) * L::PT + 4 * jb]) = w;
      }
    }
  }
  if (tid < 64) {
    // inclusive scan of the chunk's log-gates (lane owns C/64 consecutive ones)
    constexpr int E = C / 64;
    float part[E];
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      run += pf.lg[e];
      part[e] = run;
    }
    float incl = run;
#pragma unroll
    for (int off = 1; off < 64; off *= 2) {
      const float y = __shfl_up(incl, off);
      if (tid >= off) incl += y;
    }
    const float excl = incl - run;
    const float total = __shfl(incl, 63);
    const float b2last = total * kLog2e;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = tid * E + e;
      const float b2 = (excl + part[e]) * kLog2e;
      s.b2[j] = b2;
      s.lam[j] = fast_exp2(b2);
      s.kap[j] = fast_exp2(b2last - b2);
    }
    if (tid == 0) {
      s.gam = fast_exp2(b2last);
      s.lsum = total;
    }
  }
}

template <int C, int DK, typename Tout, bool STATE_PASS>
__global__ __launch_bounds__(256) void chunk_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ lg, const float *__restrict__ S0,
    float *__restrict__ ST, Tout *__restrict__ o, const WorkItem *__restrict__ items,
    const int *__restrict__ n_items, float *__restrict__ slots, float *__restrict__ slot_gamma,
    int T, int H, int DV, int n_pairs) {
  using L = BfTile<C, DK>;
  constexpr int NM = C / 16;   // 16-row tiles of the chunk
  constexpr int NKS = DK / 32; // 32-deep k-steps over d_k
  constexpr int NT = DK / 16;  // 16-row tiles of the state
  constexpr int NJS = C / 32;  // 32-deep k-steps over the chunk
  constexpr int NTILE = NM * (NM + 1) / 2;  // lower-triangular score tiles
  __shared__ BfLds<C, DK> s;

  // Block -> (pair = item * H + head, column slice). Slices of one pair are
  // placed on the same XCD (workgroups are dealt to the 8 XCDs round-robin),
  // so their shared Q/K tiles are fetched from HBM once per L2.
  const int n_slices = DV / kBfSlice;
  const int per_round = 8 * n_slices;
  const int full = (n_pairs * n_slices) / per_round * per_round;
  int pair, slice;
  const int L0 = blockIdx.x;
  if (L0 < full) {
    const int xcd = L0 % 8, kk = L0 / 8;
    slice = kk % n_slices;
    pair = (kk / n_slices) * 8 + xcd;
  } else {
    slice = L0 % n_slices;
    pair = L0 / n_slices;
  }
  const int it = pair / H, h = pair % H;
  if (items && it >= *n_items) return;
  const WorkItem w = bf_item_for(items, it, T);

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int ln = lane % 16, lg4 = lane / 16;  // MFMA lane coordinates
  const int col0 = slice * kBfSlice;          // first state column of the slice
  const int wcol = 16 * wave;                 // wavefront's columns within the slice
  const size_t dkdv = (size_t)DK * DV;

  // State slice in accumulator layout: S_acc[t][r] = S[16t + 4*lg4 + r][col0 + wcol + ln].
  f32x4 S_acc[NT];
  {
    const float *sin = nullptr;
    if (!STATE_PASS) {
      if (w.state_in >= 0) sin = slots + ((size_t)w.state_in * H + h) * dkdv;
      else if (S0) sin = S0 + ((size_t)w.seq * H + h) * dkdv;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S_acc[t][r] = sin ? sin[(size_t)(16 * t + 4 * lg4 + r) * DV + col0 + wcol + ln] : 0.f;
  }

  // Score tiles above the diagonal are never written: zero P once.
  if (!STATE_PASS) {
    for (int i = tid; i < C * L::PT / 2; i += 256) {
      reinterpret_cast<uint32_t *>(s.Phi)[i] = 0u;
      reinterpret_cast<uint32_t *>(s.Plo)[i] = 0u;
    }
  }

  float lsum = 0.f;
  BfPrefetch<C, DK, STATE_PASS> pf;
  int t0 = w.tok_begin;
  if (t0 < w.tok_end) {
    bf_load<C, DK, STATE_PASS>(pf, q, k, v, lg, t0, min(C, w.tok_end - t0), H, h, DV, col0);
    bf_store<C, DK, STATE_PASS>(pf, s);
  }
  __syncthreads();

  for (; t0 < w.tok_end; t0 += C) {
    const int n = min(C, w.tok_end - t0);
    const int t1 = t0 + C;
    if (t1 < w.tok_end)  // prefetch the next chunk into registers
      bf_load<C, DK, STATE_PASS>(pf, q, k, v, lg, t1, min(C, w.tok_end - t1), H, h, DV, col0);

    f32x4 O_acc[STATE_PASS ? 1 : NM];
    if (!STATE_PASS) {
      // ---- scores: lower-triangular 16x16 tiles of A^T = K Q^T, dealt round-robin
      for (int tile = wave; tile < NTILE; tile += 4) {
        int ti = 0, rem = tile;  // tile -> (ti, tj) with tj <= ti
        while (rem > ti) {
          rem -= ti + 1;
          ++ti;
        }
        const int tj = rem;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const u32x4 a = *reinterpret_cast<const u32x4 *>(
              &s.K[(16 * tj + ln) * L::PQ + 32 * ks + 8 * lg4]);
          const u32x4 b = *reinterpret_cast<const u32x4 *>(
              &s.Q[(16 * ti + ln) * L::PQ + 32 * ks + 8 * lg4]);
          acc = mfma16(a, b, acc);
        }
        // acc[r] = A^T[j][i] with j = 16 tj + 4 lg4 + r, i = 16 ti + ln
        const int i = 16 * ti + ln;
        const float b2i = s.b2[i];
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * tj + 4 * lg4 + r;
          p[r] = (j <= i) ? acc[r] * fast_exp2(b2i - s.b2[j]) : 0.f;
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) split_bf16(p[r], hi[r], lo[r]);
        u32x2 wh, wl;
        wh.x = hi[0] | (hi[1] << 16);
        wh.y = hi[2] | (hi[3] << 16);
        wl.x = lo[0] | (lo[1] << 16);
        wl.y = lo[2] | (lo[3] << 16);
        *reinterpret_cast<u32x2 *>(&s.Phi[i * L::PT + 16 * tj + 4 * lg4]) = wh;
        *reinterpret_cast<u32x2 *>(&s.Plo[i * L::PT + 16 * tj + 4 * lg4]) = wl;
      }

      // ---- inter-chunk read of the state: O = Q S (before this chunk's update)
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) O_acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        // B operand from the accumulators: slot 8*lg4 + r <-> d = 32ks + 4lg4 + r,
        // slot 8*lg4 + 4 + r <-> d = 32ks + 16 + 4lg4 + r.
        uint32_t h0[8], l0[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          split_bf16(S_acc[2 * ks][r], h0[r], l0[r]);
          split_bf16(S_acc[2 * ks + 1][r], h0[4 + r], l0[4 + r]);
        }
        u32x4 bh, bl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bh[e] = h0[2 * e] | (h0[2 * e + 1] << 16);
          bl[e] = l0[2 * e] | (l0[2 * e + 1] << 16);
        }
#pragma unroll
        for (int mi = 0; mi < NM; ++mi) {
          const uint16_t *qrow = &s.Q[(16 * mi + ln) * L::PQ + 32 * ks + 4 * lg4];
          const u32x2 qa = *reinterpret_cast<const u32x2 *>(qrow);
          const u32x2 qb = *reinterpret_cast<const u32x2 *>(qrow + 16);
          const u32x4 a = {qa.x, qa.y, qb.x, qb.y};
          O_acc[mi] = mfma16(a, bh, O_acc[mi]);
          O_acc[mi] = mfma16(a, bl, O_acc[mi]);
        }
      }
      // rows scale by 2^(b2_i): O_acc[mi][r] is row 16 mi + 4 lg4 + r
#pragma unroll
      for (int mi = 0; mi < NM; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) O_acc[mi][r] *= s.lam[16 * mi + 4 * lg4 + r];
    }
    __syncthreads();  // P complete

    // V fragments of this wavefront's 16 columns: slot 8 lg4 + e <-> j = 32 js + 8 lg4 + e
    u32x4 vf[NJS];
#pragma unroll
    for (int js = 0; js < NJS; ++js)
      vf[js] = *reinterpret_cast<const u32x4 *>(&s.Vt[(wcol + ln) * L::PT + 32 * js + 8 * lg4]);

    if (!STATE_PASS) {
      // ---- intra-chunk: O += P V over the causal k-steps
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) {
#pragma unroll
        for (int js = 0; js < NJS; ++js) {
          if (32 * js <= 16 * mi + 15) {
            const int off = (16 * mi + ln) * L::PT + 32 * js + 8 * lg4;
            const u32x4 ph = *reinterpret_cast<const u32x4 *>(&s.Phi[off]);
            const u32x4 pl = *reinterpret_cast<const u32x4 *>(&s.Plo[off]);
            O_acc[mi] = mfma16(ph, vf[js], O_acc[mi]);
            O_acc[mi] = mfma16(pl, vf[js], O_acc[mi]);
          }
        }
      }
      // ---- store this wavefront's 16 output columns of the valid rows
#pragma unroll
      for (int mi = 0; mi < NM; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * mi + 4 * lg4 + r;
          if (i < n)
            store_from_f32(o, ((size_t)(t0 + i) * H + h) * DV + col0 + wcol + ln, O_acc[mi][r]);
        }
    }

    // ---- state advance: S <- gamma S + K^T (kappa . V)
    const float gam = s.gam;
    lsum += s.lsum;
#pragma unroll
    for (int t = 0; t < NT; ++t) S_acc[t] *= gam;
#pragma unroll
    for (int js = 0; js < NJS; ++js) {
      u32x4 bh, bl;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        uint32_t h2[2], l2[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int e = 2 * e2 + x;
          const float kv = s.kap[32 * js + 8 * lg4 + e] * bf16_bits_to_f32(bf_elem(vf[js], e));
          split_bf16(kv, h2[x], l2[x]);
        }
        bh[e2] = h2[0] | (h2[1] << 16);
        bl[e2] = l2[0] | (l2[1] << 16);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 a =
            *reinterpret_cast<const u32x4 *>(&s.Kt[(16 * t + ln) * L::PT + 32 * js + 8 * lg4]);
        S_acc[t] = mfma16(a, bh, S_acc[t]);
        S_acc[t] = mfma16(a, bl, S_acc[t]);
      }
    }
    __syncthreads();  // everyone is done with this chunk's LDS
    if (t1 < w.tok_end) bf_store<C, DK, STATE_PASS>(pf, s);
    __syncthreads();
  }

  // ---- final state of the run
  float *sout = nullptr;
  if (STATE_PASS) {
    sout = slots + ((size_t)w.state_out * H + h) * dkdv;
    if (slice == 0 && tid == 0) slot_gamma[(size_t)w.state_out * H + h] = lsum;
  } else if (w.state_out == -1 && ST) {
    sout = ST + ((size_t)w.seq * H + h) * dkdv;
  }
  if (sout) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sout[(size_t)(16 * t + 4 * lg4 + r) * DV + col0 + wcol + ln] = S_acc[t][r];
  }
}

template <int C, int DK, typename Tout, bool SP>
static hipError_t launch_bf_t(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *g, const float *S0, float *S_T, void *o,
                              const FwdDims &d, const WorkItem *items, const int *n_items,
                              int grid_items, float *slots, float *slot_gamma,
                              hipStream_t stream) {
  const long pairs = (long)grid_items * d.H;
  const long blocks = pairs * (d.dv / kBfSlice);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_bf16_kernel<C, DK, Tout, SP>), dim3(blocks), dim3(256), 0, stream,
                     q, k, v, g, S0, S_T, static_cast<Tout *>(o), items, n_items, slots,
                     slot_gamma, d.T, d.H, d.dv, (int)pairs);
  return hipGetLastError();
}

template <int C, int DK>
static hipError_t launch_bf_c(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *g, const float *S0, float *S_T, void *o, bool out_bf16,
                              const FwdDims &d, const WorkItem *items, const int *n_items,
                              int grid_items, float *slots, float *slot_gamma, bool state_pass,
                              hipStream_t stream) {
  if (state_pass)
    return launch_bf_t<C, DK, float, true>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                           grid_items, slots, slot_gamma, stream);
  if (out_bf16)
    return launch_bf_t<C, DK, uint16_t, false>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                               grid_items, slots, slot_gamma, stream);
  return launch_bf_t<C, DK, float, false>(q, k, v, g, S0, S_T, o, d, items, n_items, grid_items,
                                          slots, slot_gamma, stream);
}

hipError_t launch_chunk_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const float *g, const float *S0, float *S_T, void *o, bool out_bf16,
                             const FwdDims &d, const WorkItem *items, const int *n_items,
                             int grid_items, float *slots, float *slot_gamma, bool state_pass,
                             hipStream_t stream) {
  // The C ABI admits chunk_size 64 only on this path: a 128-token chunk's
  // bf16 tiles (Q, K, K^T, V^T, P hi/lo) would exceed the 160 KB of LDS.
  if (d.C != 64) return hipErrorInvalidValue;
  if (d.dk == 128)
    return launch_bf_c<64, 128>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                                slots, slot_gamma, state_pass, stream);
  return launch_bf_c<64, 64>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                             slots, slot_gamma, state_pass, stream);
}

}  // namespace gla
