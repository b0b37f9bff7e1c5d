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
// its d_k x 64 fp32 state slice in the matrix-core accumulators for the whole
// run. Wavefront w owns state and output columns 16w .. 16w+15.
//
// Data movement per chunk:
//  * Q, K (C x d_k) and the V slice (C x 64) are copied HBM -> LDS with
//    buffer loads that write LDS directly (16 bytes per lane, no register
//    staging); rows past the end of the run fall outside the buffer
//    descriptor's range and arrive as zeros. Tiles are row-major with the
//    16-byte column chunks of row r XOR-swizzled by r, so that the matrix-core
//    operand reads of 16 consecutive rows hit distinct LDS banks.
//  * With chunk size 64 the tiles are double-buffered: chunk n+1 streams in
//    while chunk n computes. A 128-token chunk's tiles and P fill LDS once,
//    so that chunk size reloads after each chunk.
//  * Operands that need the chunk dimension as the reduction index (K^T for
//    the state update, V for P V and K^T V) are read with the LDS transpose
//    read (ds_read_b64_tr_b16), so no transposed copies are kept.
//  * A chunk's outputs are stored one chunk later, so their write latency
//    overlaps the next chunk's compute instead of the next load wait.
// Per chunk:
//   1. each wavefront scans the chunk's log-gates (log2 domain) into its own
//      LDS arrays: b2_i, 2^(b2_i), 2^(b2_last - b2_j);
//   2. the lower-triangular 16x16 tiles of K Q^T are spread over the four
//      wavefronts (v_mfma_f32_16x16x32_bf16), masked by 2^(b2_i - b2_j)
//      evaluated per element, split into bf16 hi + lo and written to LDS as P;
//   3. each wavefront computes its 16 output columns transposed,
//      O^T = S^T Q^T + V^T P^T, so that each lane ends up holding four
//      consecutive columns of one output row (one 16-byte store): the state
//      accumulators serve directly as the S^T operand (the reduction order of
//      Q is permuted to match their layout), and the rows of O (columns of
//      O^T) are scaled by 2^(b2_i) before P V is added;
//   4. it advances its state: S <- gamma S + K^T (kappa . V).
// Accuracy: bf16 inputs are exact operands; every value rounded on its way
// into an MFMA (P, S, kappa . V) is split into hi = bf16(x) and
// lo = bf16(x - hi) and both parts are multiplied, which keeps ~16
// significant bits with fp32 accumulation.
#include "bf16_blocks.h"

namespace gla {

template <int C, int DK, bool SP>
struct BfLds {
  static constexpr int NST = C == 64 ? 2 : 1;  // LDS stages of the Q/K/V tiles (fit in 160 KB)
  static constexpr int QR = SP ? 1 : C;                       // the state pass keeps no Q, P
  static constexpr int PP = C + 8;                            // row pitch (bf16) of P
  uint16_t q[NST][QR * DK];
  uint16_t k[NST][C * DK];
  uint16_t v[NST][C * kBfSlice];
  float lg[NST][C];
  uint16_t phi[QR * PP];
  uint16_t plo[QR * PP];
  float gb2[4][C];   // per wavefront: in-chunk prefix sums of the log-gates, log2 units
  float glam[4][C];  // 2^(b2_i), 0 from the chunk's first reset on
  float gkap[4][C];  // 2^(b2_last - b2_j), 0 before the chunk's last reset
  int grs[4][C];     // last reset at or before position i (-1: none)
};

// HBM -> LDS copies of one chunk (rows [t0, t0 + n) of the run) into stage
// `st`; every wavefront copies a quarter of each tile. The copy is issued in
// three parts (K; Q; V and the gates) spread over the previous chunk's
// compute, so the four wavefronts do not queue all their memory instructions
// on the CU's address unit at once.
// REV: the time-reversed run of the backward (rows read bottom-up, gates
// shifted by one; see W8Loader in chunk_bf16_w8.hip).
template <int C, int DK, bool SP, bool REV = false>
struct ChunkLoader {
  static constexpr int CPR = DK / 8;                  // 16-byte chunks per Q/K row
  static constexpr int QB = C * DK * 2 / 1024;        // 1 KB blocks per Q/K tile
  static_assert(QB % 4 == 0, "Q/K tile blocks split over four wavefronts");
  static constexpr int VB = C * kBfSlice * 2 / 1024;  // 1 KB blocks of the V slice (8 rows each)
  i32x4 rq, rk, rv, rg;
  uint32_t qk_row, v_row, g_row;
  int st, n_ld;
  bool active;
  static constexpr int kFar = 0x7fff0000;  // an offset past any descriptor range

  __device__ __forceinline__ void setup(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                        const float *lg, int t0, int tok_end, int H, int gts,
                                        int h, int DV, int col0, int stage, int sb = 0,
                                        int se = 0) {
    active = t0 < tok_end;
    st = stage;
    if (!active) return;
    const int n = min(C, tok_end - t0);
    n_ld = n;
    qk_row = (uint32_t)H * DK * 2;
    v_row = (uint32_t)H * DV * 2;
    g_row = (uint32_t)gts * 4;
    if constexpr (REV) {  // lowest memory row sb + se - t0 - n; gates one row later
      const size_t lo = (size_t)(sb + se - t0 - n), tok0 = lo * H + h;
      rk = make_rsrc(k + tok0 * DK, (n - 1) * qk_row + DK * 2);
      if (!SP) rq = make_rsrc(q + tok0 * DK, (n - 1) * qk_row + DK * 2);
      rv = make_rsrc(v + tok0 * DV + col0, (n - 1) * v_row + kBfSlice * 2);
      rg = make_rsrc(lg + (lo + 1) * gts + h, (n - 1) * g_row + (t0 == sb ? 0 : 4));
      return;
    }
    const size_t tok0 = (size_t)t0 * H + h;
    rk = make_rsrc(k + tok0 * DK, (n - 1) * qk_row + DK * 2);
    if (!SP) rq = make_rsrc(q + tok0 * DK, (n - 1) * qk_row + DK * 2);
    rv = make_rsrc(v + tok0 * DV + col0, (n - 1) * v_row + kBfSlice * 2);
    rg = make_rsrc(lg + (size_t)t0 * gts + h, (n - 1) * g_row + 4);
  }
  template <typename Tiles>
  __device__ __forceinline__ void qk_part(Tiles &dst, i32x4 r, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < QB / 4; ++i) {
      const int blk = wave * (QB / 4) + i;
      // the lane's LDS slot is 16-byte chunk e of the row-major tile: row
      // e / CPR, swizzled chunk e % CPR, filled from logical chunk c
      const int e = blk * 64 + lane;
      const int row = e / CPR;
      const int c = (e % CPR) ^ qk_swz<DK>(row);
      int vo = row * qk_row + c * 16;
      if constexpr (REV) vo = row < n_ld ? (n_ld - 1 - row) * qk_row + c * 16 : kFar;
      buffer_load_to_lds(r, (lds_u32 *)&dst[st][blk * 512], 16, vo, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void k_part(BfLds<C, DK, SP> &s, int wave, int lane) {
    if (active) qk_part(s.k, rk, wave, lane);
  }
  __device__ __forceinline__ void q_part(BfLds<C, DK, SP> &s, int wave, int lane) {
    if (!SP && active) qk_part(s.q, rq, wave, lane);
  }
  __device__ __forceinline__ void v_part(BfLds<C, DK, SP> &s, int wave, int lane) {
    if (!active) return;
#pragma unroll
    for (int i = 0; i < VB / 4; ++i) {
      const int blk = wave * (VB / 4) + i;
      const int r = blk * 8 + lane / 8;
      const int c = (lane % 8) ^ (r & 7);
      int vo = r * v_row + c * 16;
      if constexpr (REV) vo = r < n_ld ? (n_ld - 1 - r) * v_row + c * 16 : kFar;
      buffer_load_to_lds(rv, (lds_u32 *)&s.v[st][blk * 512], 16, vo, 0, 0, 0);
    }
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < C / 64; ++i) {
        const int j = 64 * i + lane;
        int vo = j * g_row;
        if constexpr (REV) vo = j < n_ld ? (n_ld - 1 - j) * g_row : kFar;
        buffer_load_to_lds(rg, (lds_u32 *)&s.lg[st][64 * i], 4, vo, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void all(BfLds<C, DK, SP> &s, int wave, int lane) {
    k_part(s, wave, lane);
    q_part(s, wave, lane);
    v_part(s, wave, lane);
  }
};

template <int C, int DK, typename Tout, bool SP>
struct BfRun {
  using LDS = BfLds<C, DK, SP>;
  static constexpr int NST = LDS::NST;
  static constexpr int PP = LDS::PP;
  static constexpr int NM = C / 16;                // 16-row tiles of the chunk
  static constexpr int NKS = DK / 32;              // 32-deep k-steps over d_k
  static constexpr int NT = DK / 16;               // 16-row tiles of the state
  static constexpr int NJS = C / 32;               // 32-deep k-steps over the chunk
  static constexpr int NTILE = NM * (NM + 1) / 2;  // lower-triangular score tiles
  static constexpr int E = C / 64;                 // gate positions per lane

  LDS &s;
  int wave, lane, ln, lg4, wcol;
  __device__ __forceinline__ BfRun(LDS &s_, int wave_, int lane_)
      : s(s_), wave(wave_), lane(lane_), ln(lane_ % 16), lg4(lane_ / 16), wcol(16 * wave_) {}

  // Gates of the chunk in stage st (n tokens): in-chunk prefix sums (log2
  // units) and the decay factors, into this wavefront's LDS arrays. Positions
  // past the end add 0 (a fixed decay loads its value into every position).
  // A reset gate adds 0 and cuts every product of gates that spans it (the
  // chunk decay, e^{b_i} from the first reset on, kappa_j before the last
  // one, score keys before the query's last reset).
  // Returns the chunk decay; adds the chunk's natural-log gate sum to lsum.
  __device__ __forceinline__ float gates(int st, int n, float &lsum) {
    static_assert(E == 1 || E == 2, "gate positions per lane");
    float part[E];
    bool rst[E];
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x = lane * E + e < n ? s.lg[st][lane * E + e] : 0.f;
      rst[e] = is_reset(x);
      run += rst[e] ? 0.f : x;
      part[e] = run;
    }
    // last reset at or before each position: in this lane, else in the last
    // lane before it that holds one (position j = lane E + e)
    const uint64_t m_any = __builtin_amdgcn_ballot_w64(rst[0] || rst[E - 1]);
    const uint64_t m_hi = __builtin_amdgcn_ballot_w64(rst[E - 1]);
    const int lp = last_set_upto(m_any, lane - 1 < 0 ? 0 : lane - 1);
    const int before = lane == 0 || lp < 0 ? -1 : lp * E + (E == 2 && ((m_hi >> lp) & 1));
    const int la = last_set(m_any);
    const int rl = la < 0 ? -1 : la * E + (E == 2 && ((m_hi >> la) & 1));
    const float incl = wave_inclusive_scan(run);
    const float excl = incl - run;
    const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
    const float b2last = total * kLog2e;
    int ri = before;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = lane * E + e;
      if (rst[e]) ri = j;
      const float b2 = (excl + part[e]) * kLog2e;
      s.gb2[wave][j] = b2;
      s.grs[wave][j] = ri;
      s.glam[wave][j] = ri < 0 ? fast_exp2(b2) : 0.f;
      s.gkap[wave][j] = j < rl ? 0.f : fast_exp2(b2last - b2);
    }
    lsum += rl < 0 ? total : -__builtin_huge_valf();
    return rl < 0 ? fast_exp2(b2last) : 0.f;
  }

  // Score tiles W, W+4, ... of A^T = K Q^T (compile-time list, so the tiles'
  // operand reads and MFMA chains interleave), decay-masked, split into bf16
  // hi/lo and written to P.
  template <int W>
  __device__ __forceinline__ void scores(const uint16_t *sq, const uint16_t *sk) {
    constexpr int NW = (NTILE - W + 3) / 4;  // tiles of this wavefront
    f32x4 acc[NW];
#pragma unroll
    for (int m = 0; m < NW; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int m = 0; m < NW; ++m) {
        const int tile = W + 4 * m;
        const int ti = tile_ti(tile), tj = tile_tj(tile);
        const u32x4 a =
            *reinterpret_cast<const u32x4 *>(&sk[qk_off<DK>(16 * tj + ln, 32 * ks + 8 * lg4)]);
        const u32x4 b =
            *reinterpret_cast<const u32x4 *>(&sq[qk_off<DK>(16 * ti + ln, 32 * ks + 8 * lg4)]);
        acc[m] = mfma16(a, b, acc[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < NW; ++m) {
      const int tile = W + 4 * m;
      const int ti = tile_ti(tile), tj = tile_tj(tile);
      // acc[m][r] = A^T[j][i] with j = 16 tj + 4 lg4 + r, i = 16 ti + ln
      const int i = 16 * ti + ln;
      const float b2i = s.gb2[wave][i];
      const int ri = s.grs[wave][i];  // keys before the query's last reset are cut off
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * tj + 4 * lg4 + r;
        const float d = fast_exp2(b2i - s.gb2[wave][j]);
        p[r] = (ti > tj || j <= i) && j >= ri ? acc[m][r] * d : 0.f;
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
      default: scores<3>(sq, sk); break;
    }
  }
};

template <int C, int DK, typename Tout, bool SP, bool REV = false>
__global__ __launch_bounds__(256) void chunk_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ lg, const float *__restrict__ S0,
    float *__restrict__ ST, Tout *__restrict__ o, const WorkItem *__restrict__ items,
    const int *__restrict__ n_items, float *__restrict__ slots, float *__restrict__ slot_gamma,
    int T, int H, int gts, int DV, int n_pairs) {
  using Run = BfRun<C, DK, Tout, SP>;
  using LDS = typename Run::LDS;
  constexpr int NST = Run::NST, PP = Run::PP, NM = Run::NM, NKS = Run::NKS, NT = Run::NT,
                NJS = Run::NJS;
  __shared__ LDS s;

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
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  Run R(s, wave, lane);
  const int ln = R.ln, lg4 = R.lg4, wcol = R.wcol;
  const int col0 = slice * kBfSlice;  // first state column of the slice
  const size_t dkdv = (size_t)DK * DV;

  // State slice in accumulator layout: S_acc[t][r] = S[16t + 4*lg4 + r][col0 + wcol + ln].
  f32x4 S_acc[NT];
  {
    const float *sin = nullptr;
    if (!SP) {
      if (w.state_in >= 0) sin = slots + ((size_t)w.state_in * H + h) * dkdv;
      else if (S0) sin = S0 + ((size_t)w.seq * H + h) * dkdv;
    }
    if (sin) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S_acc[t][r] = sin[(size_t)(16 * t + 4 * lg4 + r) * DV + col0 + wcol + ln];
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) S_acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Score tiles above the diagonal are never written: zero P once.
  if (!SP) {
    for (int i = tid; i < C * PP / 2; i += 256) {
      reinterpret_cast<uint32_t *>(s.phi)[i] = 0u;
      reinterpret_cast<uint32_t *>(s.plo)[i] = 0u;
    }
  }

  float lsum = 0.f;
  f32x4 O_prev[SP ? 1 : NM];
  int t_prev = -1, n_prev = 0;
  // Deferred output store of the previous chunk. O_prev[mi][r] holds
  // O[16 mi + ln][wcol + 4 lg4 + r]: one 16-byte piece of a row.
  auto store_prev = [&]() {
    if (SP || t_prev < 0) return;
    if constexpr (REV) {  // logical row t is memory row sb + se - 1 - t
      const int r0 = w.seq_begin + w.seq_end - 1 - t_prev - ln;
      Tout *ob = o + (size_t)h * DV + col0 + wcol + 4 * lg4;
#pragma unroll
      for (int mi = 0; mi < NM; ++mi)
        if (16 * mi + ln < n_prev)
          store4_from_f32(ob + (size_t)(r0 - 16 * mi) * H * DV, O_prev[mi]);
      return;
    }
    Tout *ob = o + ((size_t)(t_prev + ln) * H + h) * DV + col0 + wcol + 4 * lg4;
    const size_t rs16 = (size_t)16 * H * DV;  // 16 rows
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
      if (16 * mi + ln < n_prev) store4_from_f32(ob + mi * rs16, O_prev[mi]);
  };

  ChunkLoader<C, DK, SP, REV> ld;
  int t0 = w.tok_begin;
  ld.setup(q, k, v, lg, t0, w.tok_end, H, gts, h, DV, col0, 0, w.seq_begin, w.seq_end);
  ld.all(s, wave, lane);

  for (int ci = 0; t0 < w.tok_end; t0 += C, ++ci) {
    const int n = min(C, w.tok_end - t0);
    const int t1 = t0 + C;
    const int st = (NST == 2) ? (ci & 1) : 0;
    barrier_all();  // chunk ci's tiles are in LDS; every wavefront left chunk ci-1

    const uint16_t *sq = s.q[SP ? 0 : st];
    const uint16_t *sk = s.k[st];
    const uint16_t *sv = s.v[st];
    if (NST == 2)
      ld.setup(q, k, v, lg, t1, w.tok_end, H, gts, h, DV, col0, st ^ 1, w.seq_begin, w.seq_end);
    if (NST == 2) ld.k_part(s, wave, lane);

    const float gam = R.gates(st, n, lsum);

    f32x4 O_acc[SP ? 1 : NM];
    if (!SP) {
      // ---- scores -> P (LDS)
      R.scores_dispatch(sq, sk);
      if (NST == 2) ld.q_part(s, wave, lane);

      // ---- inter-chunk read of the state: O^T = S^T Q^T (before this chunk's update)
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) O_acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        // S^T operand from the accumulators: lane (ln, lg4) supplies column
        // wcol + ln with slot 8*lg4 + r <-> d = 32ks + 4lg4 + r and
        // slot 8*lg4 + 4 + r <-> d = 32ks + 16 + 4lg4 + r; Q^T uses the same slots.
        uint32_t sh[4], sl[4];
        split_pk_bf16(S_acc[2 * ks][0], S_acc[2 * ks][1], sh[0], sl[0]);
        split_pk_bf16(S_acc[2 * ks][2], S_acc[2 * ks][3], sh[1], sl[1]);
        split_pk_bf16(S_acc[2 * ks + 1][0], S_acc[2 * ks + 1][1], sh[2], sl[2]);
        split_pk_bf16(S_acc[2 * ks + 1][2], S_acc[2 * ks + 1][3], sh[3], sl[3]);
        const u32x4 bh = {sh[0], sh[1], sh[2], sh[3]}, bl = {sl[0], sl[1], sl[2], sl[3]};
#pragma unroll
        for (int mi = 0; mi < NM; ++mi) {
          const int r = 16 * mi + ln;
          const u32x2 qa = *reinterpret_cast<const u32x2 *>(&sq[qk_off<DK>(r, 32 * ks + 4 * lg4)]);
          const u32x2 qb =
              *reinterpret_cast<const u32x2 *>(&sq[qk_off<DK>(r, 32 * ks + 16 + 4 * lg4)]);
          const u32x4 a = {qa.x, qa.y, qb.x, qb.y};
          O_acc[mi] = mfma16(bh, a, O_acc[mi]);
          O_acc[mi] = mfma16(bl, a, O_acc[mi]);
        }
      }
      // O_acc[mi][r] = O^T[wcol + 4 lg4 + r][16 mi + ln]: row i = 16 mi + ln of O
      // scales by 2^(b2_i)
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) O_acc[mi] *= s.glam[wave][16 * mi + ln];
    }
    if (NST == 2) ld.v_part(s, wave, lane);
    barrier_lds();  // P complete

    // outputs of the previous chunk, stored now so their latency overlaps this chunk
    store_prev();

    // V fragments of this wavefront's 16 columns (transpose reads):
    // slot 8 lg4 + e <-> j = 32 js + 8 lg4 + e, column wcol + ln.
    u32x4 vf[NJS];
#pragma unroll
    for (int js = 0; js < NJS; ++js) {
      const int r0 = 32 * js + 8 * lg4 + (ln >> 2);
      const int c = wcol + 4 * (ln & 3);
      const u32x2 x0 = lds_tr16(&sv[v_off(r0, c)]);
      const u32x2 x1 = lds_tr16(&sv[v_off(r0 + 4, c)]);
      vf[js] = u32x4{x0.x, x0.y, x1.x, x1.y};
    }

    if (!SP) {
      // ---- intra-chunk: O^T += V^T P^T over the causal k-steps
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) {
#pragma unroll
        for (int js = 0; js < NJS; ++js) {
          if (32 * js <= 16 * mi + 15) {
            const int off = (16 * mi + ln) * PP + 32 * js + 8 * lg4;
            const u32x4 ph = *reinterpret_cast<const u32x4 *>(&s.phi[off]);
            const u32x4 pl = *reinterpret_cast<const u32x4 *>(&s.plo[off]);
            O_acc[mi] = mfma16(vf[js], ph, O_acc[mi]);
            O_acc[mi] = mfma16(vf[js], pl, O_acc[mi]);
          }
        }
      }
    }

    // ---- state advance: S <- gamma S + K^T (kappa . V)
#pragma unroll
    for (int t = 0; t < NT; ++t) S_acc[t] *= gam;
#pragma unroll
    for (int js = 0; js < NJS; ++js) {
      uint32_t kh[4], kl[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int j = 32 * js + 8 * lg4 + 2 * e2;
        const uint32_t vw = vf[js][e2];
        const float v0 = __uint_as_float(vw << 16), v1 = __uint_as_float(vw & 0xffff0000u);
        split_pk_bf16(s.gkap[wave][j] * v0, s.gkap[wave][j + 1] * v1, kh[e2], kl[e2]);
      }
      const u32x4 bh = {kh[0], kh[1], kh[2], kh[3]}, bl = {kl[0], kl[1], kl[2], kl[3]};
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        // A operand K^T: slot 8 lg4 + e <-> j = 32 js + 8 lg4 + e, d = 16 t + ln
        const int r0 = 32 * js + 8 * lg4 + (ln >> 2);
        const int c = 16 * t + 4 * (ln & 3);
        const u32x2 x0 = lds_tr16(&sk[qk_off<DK>(r0, c)]);
        const u32x2 x1 = lds_tr16(&sk[qk_off<DK>(r0 + 4, c)]);
        const u32x4 a = {x0.x, x0.y, x1.x, x1.y};
        S_acc[t] = mfma16(a, bh, S_acc[t]);
        S_acc[t] = mfma16(a, bl, S_acc[t]);
      }
    }

    if (!SP) {
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) O_prev[mi] = O_acc[mi];
      t_prev = t0;
      n_prev = n;
    }
    if (NST == 1 && t1 < w.tok_end) {
      barrier_lds();  // every wavefront is done with the single stage
      ld.setup(q, k, v, lg, t1, w.tok_end, H, gts, h, DV, col0, 0, w.seq_begin, w.seq_end);
      ld.all(s, wave, lane);
    }
  }

  // ---- last chunk's outputs, final state of the run
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
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sout[(size_t)(16 * t + 4 * lg4 + r) * DV + col0 + wcol + ln] = S_acc[t][r];
  }
}

template <int C, int DK, typename Tout, bool SP, bool REV = false>
static hipError_t launch_bf_t(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *g, const float *S0, float *S_T, void *o,
                              const FwdDims &d, const WorkItem *items, const int *n_items,
                              int grid_items, float *slots, float *slot_gamma,
                              hipStream_t stream) {
  const long pairs = (long)grid_items * d.H;
  const long blocks = pairs * (d.dv / kBfSlice);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_bf16_kernel<C, DK, Tout, SP, REV>), dim3(blocks), dim3(256), 0, stream,
                     q, k, v, g, S0, S_T, static_cast<Tout *>(o), items, n_items, slots,
                     slot_gamma, d.T, d.H, d.gts, d.dv, (int)pairs);
  return hipGetLastError();
}

template <int C, int DK>
static hipError_t launch_bf_c(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *g, const float *S0, float *S_T, void *o, bool out_bf16,
                              const FwdDims &d, const WorkItem *items, const int *n_items,
                              int grid_items, float *slots, float *slot_gamma, bool state_pass,
                              hipStream_t stream) {
  if (d.rev) {  // time-reversed runs of the backward: fp32 outputs, d_k in {64, 128}
    if constexpr (DK == 96) {
      return hipErrorInvalidValue;
    } else {
      if (state_pass)
        return launch_bf_t<C, DK, float, true, true>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                                     grid_items, slots, slot_gamma, stream);
      if (out_bf16) return hipErrorInvalidValue;
      return launch_bf_t<C, DK, float, false, true>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                                    grid_items, slots, slot_gamma, stream);
    }
  }
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
  // 64-token chunks run on the eight- (twelve-) wavefront kernel; this file's
  // four-wavefront kernel serves 128-token chunks (whose tiles leave no LDS for
  // more wavefronts).
  if (d.C == 64)
    return launch_chunk_bf16_c64(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                                 slots, slot_gamma, state_pass, stream);
  if (d.dot_x) return hipErrorInvalidValue;  // row dots: chunk-64 kernel only
  if (d.dk == 96)
    return launch_bf_c<128, 96>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                                slots, slot_gamma, state_pass, stream);
  if (d.dk == 128)
    return launch_bf_c<128, 128>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items,
                                 grid_items, slots, slot_gamma, state_pass, stream);
  return launch_bf_c<128, 64>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                              slots, slot_gamma, state_pass, stream);
}

}  // namespace gla
