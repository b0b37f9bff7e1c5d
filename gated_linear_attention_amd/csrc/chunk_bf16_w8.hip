// Chunked GLA forward, bf16 inputs, 64-token chunks, eight wavefronts per
// workgroup (two per SIMD).
//
// The algebra is the chunked form of Laplace 3B on AWS Trainium2
// (automationscribe.com/?p=7116), "Challenge 1", as in chunk_bf16.hip:
//   O = diag(e^{b}) Q S + ((Q K^T) .* D) V,   S <- e^{b_last} S + K^T (e^{b_last - b} . V).
//
// Decomposition: one 512-thread workgroup per (work item, head, 64-column
// slice of the state), like the four-wavefront kernel, but each wavefront
// owns half as much: wavefront (c, r) (c = w & 3, r = w >> 2) holds state rows
// [r d_k/2, (r+1) d_k/2) of columns 16c .. 16c+15 in its accumulators. Per
// chunk it
//   * computes its share of the lower-triangular score tiles into P (LDS);
//   * computes the state read over its half of d_k for all 64 rows,
//     O^T_part = S_half^T Q_half^T, and hands the rows it does not own to its
//     partner (c, 1-r) through LDS;
//   * after the one mid-chunk barrier, adds the partner's half for its own 32
//     rows, scales them by e^{b_i}, adds V^T P^T for those rows, and stores
//     them one chunk later (16-byte row pieces);
//   * advances its half of the state: S_half <- gamma S_half + K_half^T (kappa . V).
// Each wavefront's dependency chain is half as long as with four wavefronts,
// and two wavefronts per SIMD let one's MFMA, VALU and LDS work overlap the
// other's waits. Data movement (HBM -> LDS buffer loads into swizzled,
// double-buffered tiles; LDS transpose reads; hi/lo bf16 splits of P, S and
// kappa . V) is the same as in chunk_bf16.hip.
#include "bf16_blocks.h"

namespace gla {

namespace {

constexpr int kW8C = 64;      // chunk size of this kernel
constexpr int kW8Waves = 8;

template <int DK, bool SP>
struct W8Lds {
  static constexpr int C = kW8C;
  static constexpr int QR = SP ? 1 : C;
  static constexpr int PP = C + 8;  // row pitch (bf16) of P
  uint16_t q[2][QR * DK];
  uint16_t k[2][C * DK];
  uint16_t v[2][C * kBfSlice];
  float lg[2][C];
  uint16_t phi[QR * PP];
  uint16_t plo[QR * PP];
  f32x4 xbuf[SP ? 1 : kW8Waves][2][64];  // partial outputs handed to the partner wavefront
  float gb2[kW8Waves][C];   // per wavefront: in-chunk prefix sums of the log-gates, log2 units
  float glam[kW8Waves][C];  // 2^(b2_i)
  float gkap[kW8Waves][C];  // 2^(b2_last - b2_j)
};

// HBM -> LDS copy of one chunk into stage st, split in three parts over eight
// wavefronts (see ChunkLoader in chunk_bf16.hip for the swizzle).
template <int DK, bool SP>
struct W8Loader {
  static constexpr int C = kW8C;
  static constexpr int CPR = DK / 8;
  static constexpr int QB = C * DK * 2 / 1024;  // 1 KB blocks per Q/K tile (8 or 16)
  static constexpr int RPB = 1024 / (DK * 2);
  static constexpr int VB = C * kBfSlice * 2 / 1024;  // 8
  static_assert(QB % kW8Waves == 0 && VB % kW8Waves == 0, "blocks per wavefront");
  i32x4 rq, rk, rv, rg;
  uint32_t qk_row, v_row, g_row;
  int st;
  bool active;

  __device__ __forceinline__ void setup(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                        const float *lg, int t0, int tok_end, int H, int h,
                                        int DV, int col0, int stage) {
    active = t0 < tok_end;
    st = stage;
    if (!active) return;
    const int n = min(C, tok_end - t0);
    const size_t tok0 = (size_t)t0 * H + h;
    qk_row = (uint32_t)H * DK * 2;
    v_row = (uint32_t)H * DV * 2;
    g_row = (uint32_t)H * 4;
    rk = make_rsrc(k + tok0 * DK, (n - 1) * qk_row + DK * 2);
    if (!SP) rq = make_rsrc(q + tok0 * DK, (n - 1) * qk_row + DK * 2);
    rv = make_rsrc(v + tok0 * DV + col0, (n - 1) * v_row + kBfSlice * 2);
    rg = make_rsrc(lg + tok0, (n - 1) * g_row + 4);
  }
  template <typename Tiles>
  __device__ __forceinline__ void qk_part(Tiles &dst, i32x4 r, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < QB / kW8Waves; ++i) {
      const int blk = wave * (QB / kW8Waves) + i;
      const int row = blk * RPB + lane / CPR;
      const int c = (lane % CPR) ^ (row & (CPR - 1));
      buffer_load_to_lds(r, (lds_u32 *)&dst[st][blk * 512], 16, row * qk_row + c * 16, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void k_part(W8Lds<DK, SP> &s, int wave, int lane) {
    if (active) qk_part(s.k, rk, wave, lane);
  }
  __device__ __forceinline__ void q_part(W8Lds<DK, SP> &s, int wave, int lane) {
    if (!SP && active) qk_part(s.q, rq, wave, lane);
  }
  __device__ __forceinline__ void v_part(W8Lds<DK, SP> &s, int wave, int lane) {
    if (!active) return;
#pragma unroll
    for (int i = 0; i < VB / kW8Waves; ++i) {
      const int blk = wave * (VB / kW8Waves) + i;
      const int r = blk * 8 + lane / 8;
      const int c = (lane % 8) ^ (r & 7);
      buffer_load_to_lds(rv, (lds_u32 *)&s.v[st][blk * 512], 16, r * v_row + c * 16, 0, 0, 0);
    }
    if (wave == 0) buffer_load_to_lds(rg, (lds_u32 *)&s.lg[st][0], 4, lane * g_row, 0, 0, 0);
  }
};

template <int DK, bool SP>
struct W8Wave {
  using LDS = W8Lds<DK, SP>;
  static constexpr int C = kW8C;
  static constexpr int PP = LDS::PP;
  static constexpr int NTILE = 10;     // lower-triangular 16x16 score tiles of a 64-token chunk
  static constexpr int NKS = DK / 32;  // 32-deep k-steps over d_k (scores)
  LDS &s;
  int wave, lane, ln, lg4;
  __device__ __forceinline__ W8Wave(LDS &s_, int w, int l)
      : s(s_), wave(w), lane(l), ln(l % 16), lg4(l / 16) {}

  __device__ __forceinline__ float gates(int st, float &lsum) {
    const float x = s.lg[st][lane];
    const float incl = wave_inclusive_scan(x);
    const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
    const float b2last = total * kLog2e;
    const float b2 = incl * kLog2e;
    s.gb2[wave][lane] = b2;
    s.glam[wave][lane] = fast_exp2(b2);
    s.gkap[wave][lane] = fast_exp2(b2last - b2);
    lsum += total;
    return fast_exp2(b2last);
  }

  // Score tiles W and W + 8 of A^T = K Q^T -> decay mask -> bf16 hi/lo P.
  // All operand reads are issued before the first MFMA.
  template <int W>
  __device__ __forceinline__ void scores(const uint16_t *sq, const uint16_t *sk) {
    constexpr int NW = W + 8 < NTILE ? 2 : 1;
    u32x4 a[NW][NKS], b[NW][NKS];
    f32x4 g4[NW];
    float b2i[NW];
#pragma unroll
    for (int m = 0; m < NW; ++m) {
      const int tile = W + 8 * m;
      const int ti = tile_ti(tile), tj = tile_tj(tile);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        a[m][ks] =
            *reinterpret_cast<const u32x4 *>(&sk[qk_off<DK>(16 * tj + ln, 32 * ks + 8 * lg4)]);
        b[m][ks] =
            *reinterpret_cast<const u32x4 *>(&sq[qk_off<DK>(16 * ti + ln, 32 * ks + 8 * lg4)]);
      }
      b2i[m] = s.gb2[wave][16 * ti + ln];
      g4[m] = *reinterpret_cast<const f32x4 *>(&s.gb2[wave][16 * tj + 4 * lg4]);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[NW];
#pragma unroll
    for (int m = 0; m < NW; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int m = 0; m < NW; ++m) acc[m] = mfma16(a[m][ks], b[m][ks], acc[m]);
#pragma unroll
    for (int m = 0; m < NW; ++m) {
      const int tile = W + 8 * m;
      const int ti = tile_ti(tile), tj = tile_tj(tile);
      const int i = 16 * ti + ln;  // acc[m][r] = A^T[16 tj + 4 lg4 + r][i]
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * tj + 4 * lg4 + r;
        // masked entries (j > i) take 2^-inf = 0; the select is on the exponent
        const float e = (ti > tj || j <= i) ? b2i[m] - g4[m][r] : -__builtin_huge_valf();
        p[r] = acc[m][r] * fast_exp2(e);
      }
      uint32_t h0, l0, h1, l1;
      split_pk_bf16(p[0], p[1], h0, l0);
      split_pk_bf16(p[2], p[3], h1, l1);
      const u32x2 wh = {h0, h1}, wl = {l0, l1};
      *reinterpret_cast<u32x2 *>(&s.phi[i * PP + 16 * tj + 4 * lg4]) = wh;
      *reinterpret_cast<u32x2 *>(&s.plo[i * PP + 16 * tj + 4 * lg4]) = wl;
    }
  }
  __device__ __forceinline__ void scores_dispatch(const uint16_t *sq, const uint16_t *sk) {
    switch (wave) {
      case 0: scores<0>(sq, sk); break;
      case 1: scores<1>(sq, sk); break;
      case 2: scores<2>(sq, sk); break;
      case 3: scores<3>(sq, sk); break;
      case 4: scores<4>(sq, sk); break;
      case 5: scores<5>(sq, sk); break;
      case 6: scores<6>(sq, sk); break;
      default: scores<7>(sq, sk); break;
    }
  }
};

}  // namespace

template <int DK, typename Tout, bool SP>
__global__ __launch_bounds__(512) void chunk_bf16_w8_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ lg, const float *__restrict__ S0,
    float *__restrict__ ST, Tout *__restrict__ o, const WorkItem *__restrict__ items,
    const int *__restrict__ n_items, float *__restrict__ slots, float *__restrict__ slot_gamma,
    int T, int H, int DV, int n_pairs) {
  using Wv = W8Wave<DK, SP>;
  using LDS = typename Wv::LDS;
  constexpr int C = kW8C;
  constexpr int PP = LDS::PP;
  constexpr int HALF = DK / 2;    // state rows per wavefront
  constexpr int NTH = DK / 32;    // 16-row state tiles per wavefront
  constexpr int NKH = DK / 64;    // 32-deep k-steps over the wavefront's half of d_k
  constexpr int NJS = C / 32;     // 32-deep k-steps over the chunk
  __shared__ LDS s;

  // Block -> (pair = item * H + head, column slice); slices of a pair share an XCD.
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
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  Wv R(s, wave, lane);
  const int ln = R.ln, lg4 = R.lg4;
  const int cg = wave & 3, rh = wave >> 2;  // column group, d_k half / row half
  const int wcol = 16 * cg;
  const int drow0 = HALF * rh;              // first state row of this wavefront
  const int col0 = slice * kBfSlice;
  const size_t dkdv = (size_t)DK * DV;

  // State half in accumulator layout: S_acc[t][r] = S[drow0 + 16t + 4 lg4 + r][col0 + wcol + ln].
  f32x4 S_acc[NTH];
  {
    const float *sin = nullptr;
    if (!SP) {
      if (w.state_in >= 0) sin = slots + ((size_t)w.state_in * H + h) * dkdv;
      else if (S0) sin = S0 + ((size_t)w.seq * H + h) * dkdv;
    }
    if (sin) {
#pragma unroll
      for (int t = 0; t < NTH; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S_acc[t][r] = sin[(size_t)(drow0 + 16 * t + 4 * lg4 + r) * DV + col0 + wcol + ln];
    } else {
#pragma unroll
      for (int t = 0; t < NTH; ++t) S_acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  if (!SP) {
    for (int i = tid; i < C * PP / 2; i += 512) {
      reinterpret_cast<uint32_t *>(s.phi)[i] = 0u;
      reinterpret_cast<uint32_t *>(s.plo)[i] = 0u;
    }
  }

  float lsum = 0.f;
  // O_prev[m][r] = O[16 (2 rh + m) + ln][wcol + 4 lg4 + r] of the previous chunk.
  f32x4 O_prev[2];
  int t_prev = -1, n_prev = 0;
  auto store_prev = [&]() {
    if (SP || t_prev < 0) return;
    Tout *ob = o + ((size_t)(t_prev + 32 * rh + ln) * H + h) * DV + col0 + wcol + 4 * lg4;
    const size_t rs16 = (size_t)16 * H * DV;
#pragma unroll
    for (int m = 0; m < 2; ++m)
      if (32 * rh + 16 * m + ln < n_prev) store4_from_f32(ob + m * rs16, O_prev[m]);
  };

  W8Loader<DK, SP> ld;
  int t0 = w.tok_begin;
  ld.setup(q, k, v, lg, t0, w.tok_end, H, h, DV, col0, 0);
  ld.k_part(s, wave, lane);
  ld.q_part(s, wave, lane);
  ld.v_part(s, wave, lane);

  for (int ci = 0; t0 < w.tok_end; t0 += C, ++ci) {
    const int n = min(C, w.tok_end - t0);
    const int st = ci & 1;
    barrier_all();  // chunk ci's tiles are in LDS; every wavefront left chunk ci-1

    const uint16_t *sq = s.q[SP ? 0 : st];
    const uint16_t *sk = s.k[st];
    const uint16_t *sv = s.v[st];
    ld.setup(q, k, v, lg, t0 + C, w.tok_end, H, h, DV, col0, st ^ 1);
    ld.k_part(s, wave, lane);

    const float gam = R.gates(st, lsum);

    f32x4 own[2];
    if (!SP) {
      R.scores_dispatch(sq, sk);
      ld.q_part(s, wave, lane);

      // ---- state read over this wavefront's half of d_k, all 64 rows:
      // part[mi][r] = sum over d in the half of S[d][wcol + 4 lg4 + r] Q[16 mi + ln][d]
      f32x4 part[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) part[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
      u32x4 qf[NKH][4];
#pragma unroll
      for (int ks = 0; ks < NKH; ++ks) {
        const int d0 = drow0 + 32 * ks;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const int r = 16 * mi + ln;
          const u32x2 qa = *reinterpret_cast<const u32x2 *>(&sq[qk_off<DK>(r, d0 + 4 * lg4)]);
          const u32x2 qb = *reinterpret_cast<const u32x2 *>(&sq[qk_off<DK>(r, d0 + 16 + 4 * lg4)]);
          qf[ks][mi] = u32x4{qa.x, qa.y, qb.x, qb.y};
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < NKH; ++ks) {
        // slot 8 lg4 + r <-> d = drow0 + 32 ks + 4 lg4 + r,
        // slot 8 lg4 + 4 + r <-> d = drow0 + 32 ks + 16 + 4 lg4 + r
        uint32_t sh[4], sl[4];
        split_pk_bf16(S_acc[2 * ks][0], S_acc[2 * ks][1], sh[0], sl[0]);
        split_pk_bf16(S_acc[2 * ks][2], S_acc[2 * ks][3], sh[1], sl[1]);
        split_pk_bf16(S_acc[2 * ks + 1][0], S_acc[2 * ks + 1][1], sh[2], sl[2]);
        split_pk_bf16(S_acc[2 * ks + 1][2], S_acc[2 * ks + 1][3], sh[3], sl[3]);
        const u32x4 bh = {sh[0], sh[1], sh[2], sh[3]}, bl = {sl[0], sl[1], sl[2], sl[3]};
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) part[mi] = mfma16(bh, qf[ks][mi], part[mi]);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) part[mi] = mfma16(bl, qf[ks][mi], part[mi]);
      }
      // rows of the partner's half go through LDS
#pragma unroll
      for (int m = 0; m < 2; ++m) s.xbuf[wave][m][lane] = part[2 * (1 - rh) + m];
#pragma unroll
      for (int m = 0; m < 2; ++m) own[m] = part[2 * rh + m];
    }
    ld.v_part(s, wave, lane);
    barrier_lds();  // P and the partial outputs are complete

    store_prev();

    // V fragments (transpose reads): slot 8 lg4 + e <-> j = 32 js + 8 lg4 + e, column wcol + ln
    u32x4 vf[NJS];
#pragma unroll
    for (int js = 0; js < NJS; ++js) {
      const int r0 = 32 * js + 8 * lg4 + (ln >> 2);
      const int c = wcol + 4 * (ln & 3);
      const u32x2 x0 = lds_tr16(&sv[v_off(r0, c)]);
      const u32x2 x1 = lds_tr16(&sv[v_off(r0 + 4, c)]);
      vf[js] = u32x4{x0.x, x0.y, x1.x, x1.y};
    }

    // operands of P V and of the state update, all issued before the MFMAs
    u32x4 pf_h[2][NJS], pf_l[2][NJS];
    f32x4 xp[2];
    float lam[2];
    if (!SP) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int mi = 2 * rh + m;
        xp[m] = s.xbuf[wave ^ 4][m][lane];
        lam[m] = s.glam[wave][16 * mi + ln];
#pragma unroll
        for (int js = 0; js < NJS; ++js) {
          if (32 * js <= 16 * mi + 15) {
            const int off = (16 * mi + ln) * PP + 32 * js + 8 * lg4;
            pf_h[m][js] = *reinterpret_cast<const u32x4 *>(&s.phi[off]);
            pf_l[m][js] = *reinterpret_cast<const u32x4 *>(&s.plo[off]);
          }
        }
      }
    }
    u32x4 kt[NJS][NTH];
    f32x4 kap[NJS][2];
#pragma unroll
    for (int js = 0; js < NJS; ++js) {
#pragma unroll
      for (int t = 0; t < NTH; ++t) {
        // A operand K^T: slot 8 lg4 + e <-> j = 32 js + 8 lg4 + e, d = drow0 + 16 t + ln
        const int r0 = 32 * js + 8 * lg4 + (ln >> 2);
        const int c = drow0 + 16 * t + 4 * (ln & 3);
        const u32x2 x0 = lds_tr16(&sk[qk_off<DK>(r0, c)]);
        const u32x2 x1 = lds_tr16(&sk[qk_off<DK>(r0 + 4, c)]);
        kt[js][t] = u32x4{x0.x, x0.y, x1.x, x1.y};
      }
      kap[js][0] = *reinterpret_cast<const f32x4 *>(&s.gkap[wave][32 * js + 8 * lg4]);
      kap[js][1] = *reinterpret_cast<const f32x4 *>(&s.gkap[wave][32 * js + 8 * lg4 + 4]);
    }
    __builtin_amdgcn_sched_barrier(0);

    if (!SP) {
      // own rows: partner's half of the state read, scale by 2^(b2_i), then V^T P^T
#pragma unroll
      for (int m = 0; m < 2; ++m) own[m] = (own[m] + xp[m]) * lam[m];
#pragma unroll
      for (int js = 0; js < NJS; ++js) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int mi = 2 * rh + m;
          if (32 * js <= 16 * mi + 15) own[m] = mfma16(vf[js], pf_h[m][js], own[m]);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int mi = 2 * rh + m;
          if (32 * js <= 16 * mi + 15) own[m] = mfma16(vf[js], pf_l[m][js], own[m]);
        }
      }
    }

    // ---- state advance for this half: S <- gamma S + K_half^T (kappa . V)
#pragma unroll
    for (int t = 0; t < NTH; ++t) S_acc[t] *= gam;
#pragma unroll
    for (int js = 0; js < NJS; ++js) {
      uint32_t kh[4], kl[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t vw = vf[js][e2];
        const float v0 = __uint_as_float(vw << 16), v1 = __uint_as_float(vw & 0xffff0000u);
        const f32x4 &kk = kap[js][e2 >> 1];
        split_pk_bf16(kk[2 * (e2 & 1)] * v0, kk[2 * (e2 & 1) + 1] * v1, kh[e2], kl[e2]);
      }
      const u32x4 bh = {kh[0], kh[1], kh[2], kh[3]}, bl = {kl[0], kl[1], kl[2], kl[3]};
#pragma unroll
      for (int t = 0; t < NTH; ++t) S_acc[t] = mfma16(kt[js][t], bh, S_acc[t]);
#pragma unroll
      for (int t = 0; t < NTH; ++t) S_acc[t] = mfma16(kt[js][t], bl, S_acc[t]);
    }

    if (!SP) {
      O_prev[0] = own[0];
      O_prev[1] = own[1];
      t_prev = t0;
      n_prev = n;
    }
  }

  store_prev();
  float *sout = nullptr;
  if (SP) {
    sout = slots + ((size_t)w.state_out * H + h) * dkdv;
    if (slice == 0 && tid == 0) slot_gamma[(size_t)w.state_out * H + h] = lsum;
  } else if (w.state_out == -1 && ST) {
    sout = ST + ((size_t)w.seq * H + h) * dkdv;
  }
  if (sout) {
#pragma unroll
    for (int t = 0; t < NTH; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sout[(size_t)(drow0 + 16 * t + 4 * lg4 + r) * DV + col0 + wcol + ln] = S_acc[t][r];
  }
}

template <int DK, typename Tout, bool SP>
static hipError_t launch_w8_t(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *g, const float *S0, float *S_T, void *o,
                              const FwdDims &d, const WorkItem *items, const int *n_items,
                              int grid_items, float *slots, float *slot_gamma,
                              hipStream_t stream) {
  const long pairs = (long)grid_items * d.H;
  const long blocks = pairs * (d.dv / kBfSlice);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_bf16_w8_kernel<DK, Tout, SP>), dim3(blocks), dim3(512), 0, stream,
                     q, k, v, g, S0, S_T, static_cast<Tout *>(o), items, n_items, slots,
                     slot_gamma, d.T, d.H, d.dv, (int)pairs);
  return hipGetLastError();
}

template <int DK>
static hipError_t launch_w8_d(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *g, const float *S0, float *S_T, void *o, bool out_bf16,
                              const FwdDims &d, const WorkItem *items, const int *n_items,
                              int grid_items, float *slots, float *slot_gamma, bool state_pass,
                              hipStream_t stream) {
  if (state_pass)
    return launch_w8_t<DK, float, true>(q, k, v, g, S0, S_T, o, d, items, n_items, grid_items,
                                        slots, slot_gamma, stream);
  if (out_bf16)
    return launch_w8_t<DK, uint16_t, false>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                            grid_items, slots, slot_gamma, stream);
  return launch_w8_t<DK, float, false>(q, k, v, g, S0, S_T, o, d, items, n_items, grid_items,
                                       slots, slot_gamma, stream);
}

hipError_t launch_chunk_bf16_c64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const float *g, const float *S0, float *S_T, void *o,
                                 bool out_bf16, const FwdDims &d, const WorkItem *items,
                                 const int *n_items, int grid_items, float *slots,
                                 float *slot_gamma, bool state_pass, hipStream_t stream) {
  if (d.dk == 128)
    return launch_w8_d<128>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                            slots, slot_gamma, state_pass, stream);
  return launch_w8_d<64>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items, slots,
                         slot_gamma, state_pass, stream);
}

}  // namespace gla
