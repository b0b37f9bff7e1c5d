// Chunked GLA forward for bf16 inputs on the CDNA4 matrix cores: 64-token
// chunks, eight wavefronts per workgroup (two per SIMD).
//
// Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), "Challenge 1":
// within each chunk the output is decay-masked linear attention over the
// chunk plus the query's read of the running state; chunks are independent
// except for the state, which advances by the decay compounded over the
// chunk. With b_i the in-chunk inclusive cumulative log-gate:
//
//   O = diag(e^{b}) Q S + ((Q K^T) .* D) V,   D_ij = e^{b_i - b_j} (j <= i)
//   S <- e^{b_last} S + K^T (e^{b_last - b} . V)
//
// D is evaluated per element as the exponential of a difference (never as a
// product e^{b_i} e^{-b_j}, which overflows for strong decay). The page's
// chunks are 128 tokens, matched to Trainium2's 128 SBUF partitions; here the
// tile is 64 tokens (a 128-token chunk is two 64-token chunks in exact
// arithmetic), which lets the Q, K and V tiles double-buffer in LDS.
//
// Decomposition: one 512-thread workgroup per (work item, head, 64-column
// slice of the state); a work item is a run of one sequence's tokens, walked
// chunk by chunk with the fp32 state slice in the matrix-core accumulators for
// the whole run. Wavefront (c, r) (c = w & 3, r = w >> 2) holds state rows
// [r d_k/2, (r+1) d_k/2) of columns 16c .. 16c+15. Per chunk it
//   * computes its share of the lower-triangular score tiles into P (LDS);
//   * computes the state read over its half of d_k for all 64 rows,
//     O^T_part = S_half^T Q_half^T, and hands the rows it does not own to its
//     partner (c, 1-r) through LDS;
//   * after the one mid-chunk barrier, adds the partner's half for its own 32
//     rows, scales them by e^{b_i}, adds V^T P^T for those rows, and stores
//     them at the chunk's end (16-byte row pieces);
//   * advances its half of the state: S_half <- gamma S_half + K_half^T (kappa . V).
// Each wavefront's dependency chain is short, and two wavefronts per SIMD let
// one's MFMA, VALU and LDS work overlap the other's waits.
//
// Data movement: Q, K (64 x d_k) and the V slice are copied HBM -> LDS with
// buffer loads that write LDS directly (16 bytes per lane, no register
// staging); rows past the end of the run fall outside the buffer descriptor's
// range and arrive as zeros. Tiles are row-major with the 16-byte column
// chunks of row r XOR-swizzled by r, so that operand reads of 16 consecutive
// rows hit distinct LDS banks, and double-buffered: chunk n+1 streams in while
// chunk n computes. Operands that need the chunk dimension as the reduction
// index (K^T for the state update, V for P V) are read with the LDS transpose
// read (ds_read_b64_tr_b16), so no transposed copies are kept.
//
// Accuracy: bf16 inputs are exact operands; every value rounded on its way
// into an MFMA (P, S, kappa . V) is split into hi = bf16(x) and lo =
// bf16(x - hi) and both parts are multiplied, which keeps about 16 significant
// bits with fp32 accumulation.
//
// The same kernel serves the 96 x 192 heads of Laplace 3B ("GLA mixer") with
// six column groups: twelve wavefronts (three per SIMD) over a 96-column slice,
// so a head is two slices. Each wavefront then holds 48 state rows, and the
// state read over its half of d_k takes one 32-deep and one 16-deep
// matrix-core step; ten wavefronts compute one score tile each.
#include "bf16_blocks.h"
#include "tile_loader.h"

namespace gla {

namespace {

// NCG column groups of 16: 2 NCG wavefronts over a slice of 16 NCG state columns.
template <int DK, int NCG, bool SP>
struct W8Lds {
  static constexpr int C = kW8C;
  static constexpr int NW = 2 * NCG;  // wavefronts
  static constexpr int SW = 16 * NCG; // state columns of the slice
  static constexpr int QR = SP ? 1 : C;
  static constexpr int PP = C + 8;  // row pitch (bf16) of P
  uint16_t q[2][QR * DK];
  uint16_t k[2][C * DK];
  uint16_t v[2][C * SW];
  uint16_t phi[QR * PP];
  uint16_t plo[QR * PP];
  f32x4 xbuf[SP ? 1 : NW][2][64];  // partial outputs handed to the partner wavefront
  u32x4 kvx[NW][2][64];            // kappa . V (hi, lo) for the partner's 32 keys
  float lgb[3][C];                 // log-gates, loaded two chunks ahead
  float gb2[NW][C];   // per wavefront: in-chunk prefix sums of the log-gates, log2 units
  float glam[NW][C];  // 2^(b2_i), 0 from the chunk's first reset on
  float gkap[NW][C];  // 2^(b2_last - b2_j), 0 before the chunk's last reset
  int grs[NW][C];     // last reset at or before position i (-1: none)
};

template <int DK, int NCG, bool SP>
struct W8Wave {
  using LDS = W8Lds<DK, NCG, SP>;
  static constexpr int C = kW8C;
  static constexpr int PP = LDS::PP;
  static constexpr int NTILE = 10;     // lower-triangular 16x16 score tiles of a 64-token chunk
  static constexpr int NKS = DK / 32;  // 32-deep k-steps over d_k (scores)
  LDS &s;
  int wave, lane, ln, lg4;
  __device__ __forceinline__ W8Wave(LDS &s_, int w, int l)
      : s(s_), wave(w), lane(l), ln(l % 16), lg4(l / 16) {}

  // x = this lane's log-gate (0 past the end of the run); returns the chunk
  // decay. A reset gate enters the prefix sums as 0 and cuts every product of
  // gates that spans it: the chunk decay and e^{b_i} are 0 from the chunk's
  // first reset on, kappa_j = 0 for keys before its last reset, and the score
  // mask drops keys before the query's last reset (grs, -1 without one).
  // Without resets the values are those of the plain scan.
  __device__ __forceinline__ float gates(float x, float &lsum) {
    const bool rst = is_reset(x);
    const uint64_t rm = __builtin_amdgcn_ballot_w64(rst);
    const float incl = wave_inclusive_scan(rst ? 0.f : x);
    const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
    const float b2last = total * kLog2e;
    const float b2 = incl * kLog2e;
    const int ri = last_set_upto(rm, lane), rl = last_set(rm);
    s.gb2[wave][lane] = b2;
    s.grs[wave][lane] = ri;
    s.glam[wave][lane] = ri < 0 ? fast_exp2(b2) : 0.f;
    s.gkap[wave][lane] = lane < rl ? 0.f : fast_exp2(b2last - b2);
    lsum += rl < 0 ? total : -__builtin_huge_valf();
    return rl < 0 ? fast_exp2(b2last) : 0.f;
  }

  // One 16x16 score tile of A^T = K Q^T (rows: keys 16 tj.., columns: queries
  // 16 ti..), in three stages so that a caller can interleave them with other
  // work: operand reads, the MFMA chain, then decay mask -> bf16 hi/lo P.
  struct TileOps {
    u32x4 a[NKS], b[NKS];
    float b2i;
    int rq;  // the query's last reset in the chunk (-1: none)
    f32x4 g4;
  };
  __device__ __forceinline__ void tile_read(TileOps &t, const uint16_t *sq, const uint16_t *sk,
                                            int ti, int tj) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      t.a[ks] = *reinterpret_cast<const u32x4 *>(&sk[qk_off<DK>(16 * tj + ln, 32 * ks + 8 * lg4)]);
      t.b[ks] = *reinterpret_cast<const u32x4 *>(&sq[qk_off<DK>(16 * ti + ln, 32 * ks + 8 * lg4)]);
    }
    t.b2i = s.gb2[wave][16 * ti + ln];
    t.rq = s.grs[wave][16 * ti + ln];
    t.g4 = *reinterpret_cast<const f32x4 *>(&s.gb2[wave][16 * tj + 4 * lg4]);
  }
  __device__ __forceinline__ f32x4 tile_mma(const TileOps &t) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) acc = mfma16(t.a[ks], t.b[ks], acc);
    return acc;
  }
  // madd[r] = 0 where key j = 16 tj + 4 lg4 + r may attend query i = 16 ti + ln
  // (j <= i, and j at or after the query's last reset rq; rq = -1 without
  // one), -inf where masked; the decay factor is 2^(b2_i - b2_j + madd).
  __device__ __forceinline__ f32x4 tile_mask(int ti, int tj, int rq = -1) const {
    f32x4 m;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * tj + 4 * lg4 + r;
      m[r] = (ti > tj || j <= 16 * ti + ln) && j >= rq ? 0.f : -__builtin_huge_valf();
    }
    return m;
  }
  __device__ __forceinline__ void tile_store(const f32x4 &acc, const TileOps &t, const f32x4 &madd,
                                             int ti, int tj) {
    const int i = 16 * ti + ln;  // acc[r] = A^T[16 tj + 4 lg4 + r][i]
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = acc[r] * fast_exp2(t.b2i - t.g4[r] + madd[r]);
    uint32_t h0, l0, h1, l1;
    split_pk_bf16(p[0], p[1], h0, l0);
    split_pk_bf16(p[2], p[3], h1, l1);
    const u32x2 wh = {h0, h1}, wl = {l0, l1};
    *reinterpret_cast<u32x2 *>(&s.phi[i * PP + 16 * tj + 4 * lg4]) = wh;
    *reinterpret_cast<u32x2 *>(&s.plo[i * PP + 16 * tj + 4 * lg4]) = wl;
  }
};

}  // namespace

// DOT: also the row dot products of the outputs with x (a bf16 tensor of the
// outputs' shape): each wavefront sums o * x over its 16 columns per row and
// writes part[((slice * NCG + column group) * H + h) * part_stride + token]
// (part_stride = tokens; a wavefront's 16 rows are 64 contiguous bytes).
//
// Head groups (hg > 1): q, k, S0, S_T and the state slots have H heads, and
// v, the gates and the outputs H / hg: head h reads values and gates of head
// h / hg and writes its outputs to o (h % hg == 0) or o2 (otherwise). The
// backward uses hg = 2 to run a forward whose 192-dim keys are split into two
// 96-dim halves (the scores and the state rows separate over key dimensions,
// so the two halves' outputs add): a [.., 192] tensor is [.., 2, 96], and a
// 192 x 96 state is two stacked 96 x 96 ones.
template <int DK, int NCG, typename Tout, bool SP, bool REV = false, bool DOT = false>
__global__ __launch_bounds__(128 * NCG) void chunk_bf16_w8_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ lg, const float *__restrict__ S0,
    float *__restrict__ ST, Tout *__restrict__ o, const WorkItem *__restrict__ items,
    const int *__restrict__ n_items, float *__restrict__ slots, float *__restrict__ slot_gamma,
    int T, int H, int gts, int DV, int n_pairs, const uint16_t *__restrict__ xd,
    float *__restrict__ dpart, long part_stride, int hg, Tout *__restrict__ o2) {
  using Wv = W8Wave<DK, NCG, SP>;
  using LDS = typename Wv::LDS;
  using Loader = W8Loader<DK, NCG, SP, REV>;
  constexpr int C = kW8C;
  constexpr int PP = LDS::PP;
  constexpr int SW = LDS::SW;
  constexpr int HALF = DK / 2;    // state rows per wavefront
  constexpr int NTH = DK / 32;    // 16-row state tiles per wavefront
  constexpr int NKH = DK / 64;    // 32-deep k-steps over the wavefront's half of d_k
  constexpr bool QREM = DK % 64 != 0;  // and one 16-deep step (d_k = 96)
  __shared__ LDS s;

  // Block -> (pair = item * H + head, column slice); slices of a pair share an XCD.
  const int n_slices = DV / SW;
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
  const int HR = H / hg, hr = h / hg;             // values', gates' and outputs' heads
  Tout *const ow = hg > 1 && h % hg ? o2 : o;     // this head's output tensor
  if (items && it >= *n_items) return;
  const WorkItem w = bf_item_for(items, it, T);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  Wv R(s, wave, lane);
  // Row half 1 has the longer chain per chunk (with four column groups,
  // wavefronts 4 and 5 also compute the two extra score tiles); let the SIMD
  // arbiter prefer it over row half 0, which waits at the mid-chunk barrier
  // otherwise.
  if constexpr (NCG == 4) {
    if (wave >= 6)
      __builtin_amdgcn_s_setprio(2);
    else if (wave >= 4)
      __builtin_amdgcn_s_setprio(3);
  } else {
    if (wave >= NCG) __builtin_amdgcn_s_setprio(2);
  }
  const int ln = R.ln, lg4 = R.lg4;
  int cg, rh;  // column group, d_k half / row half
  if constexpr (NCG == 4) {
    cg = wave & 3;
    rh = wave >> 2;
  } else {
    cg = wave % NCG;
    rh = wave / NCG;
  }
  const int pw = NCG == 4 ? (wave ^ 4) : (rh ? wave - NCG : wave + NCG);  // partner (cg, 1 - rh)
  const int wcol = 16 * cg;
  const int drow0 = HALF * rh;              // first state row of this wavefront
  const int col0 = slice * SW;
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
    for (int i = tid; i < C * PP / 2; i += 128 * NCG) {
      reinterpret_cast<uint32_t *>(s.phi)[i] = 0u;
      reinterpret_cast<uint32_t *>(s.plo)[i] = 0u;
    }
  }

  float lsum = 0.f;
  // Output row blocks (16 rows) owned by this wavefront: rows 0..15 and
  // 48..63 for row half 0, rows 16..47 for row half 1, so that both halves
  // see the same number of key blocks in P V.
  const int mi0 = rh, mi1 = 3 - rh;  // (0, 3) or (1, 2)
  // own[m][r] = O[16 mi_m + ln][wcol + 4 lg4 + r]: 16-byte row pieces, stored at
  // the end of the chunk. Loads and stores share one counter and need not
  // complete in order, so this wavefront's loads are waited for first (issued
  // long before, they have landed); the barrier that opens the next chunk then
  // lets just these stores stay in flight.
  const size_t rs16 = (size_t)16 * HR * DV;
  auto mem_row = [&](int t) -> size_t {
    return (size_t)(REV ? w.seq_begin + w.seq_end - 1 - t : t);
  };
  auto store_out = [&](int tc, int nc, const f32x4 (&own)[2], const u32x2 (&xv)[2]) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (DOT) {  // partial row dot products: 16 columns, reduced over lg4
      float dsum[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float x0 = __uint_as_float(xv[m].x << 16), x1 = __uint_as_float(xv[m].x & 0xffff0000u);
        const float x2 = __uint_as_float(xv[m].y << 16), x3 = __uint_as_float(xv[m].y & 0xffff0000u);
        float d = own[m][0] * x0 + own[m][1] * x1 + own[m][2] * x2 + own[m][3] * x3;
        // the sum over the four lane groups of the row, in registers: swapping a
        // value with itself across 16-lane rows (then 32-lane halves) and adding
        // the two results gives d[l] + d[l ^ 16] (then + d[l ^ 32]) in every lane
        const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(d), __float_as_uint(d),
                                                          false, false);
        d = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
        const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(d), __float_as_uint(d),
                                                          false, false);
        dsum[m] = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
      }
      float *pp = dpart + ((size_t)(slice * NCG + cg) * H + h) * part_stride;
      if (lg4 == 0) {
        if (16 * mi0 + ln < nc) pp[mem_row(tc + 16 * mi0 + ln)] = dsum[0];
        if (16 * mi1 + ln < nc) pp[mem_row(tc + 16 * mi1 + ln)] = dsum[1];
      }
    }
    if constexpr (REV) {  // logical row t is memory row sb + se - 1 - t
      const int se1 = w.seq_begin + w.seq_end - 1 - tc - ln;
      Tout *ob = ow + ((size_t)hr) * DV + col0 + wcol + 4 * lg4;
      if (16 * mi0 + ln < nc) store4_from_f32(ob + (size_t)(se1 - 16 * mi0) * HR * DV, own[0]);
      if (16 * mi1 + ln < nc) store4_from_f32(ob + (size_t)(se1 - 16 * mi1) * HR * DV, own[1]);
    } else {
      Tout *ob = ow + ((size_t)(tc + ln) * HR + hr) * DV + col0 + wcol + 4 * lg4;
      if (16 * mi0 + ln < nc) store4_from_f32(ob + mi0 * rs16, own[0]);
      if (16 * mi1 + ln < nc) store4_from_f32(ob + mi1 * rs16, own[1]);
    }
  };



  Loader ld;
  int t0 = w.tok_begin;
  ld.init(q, k, v, lg, t0, H, HR, gts, h, hr, DV, col0, w.seq_begin, w.seq_end);
  ld.next(t0, w.tok_end, 0);
  ld.k_part(s, wave, lane);
  ld.q_part(s, wave, lane);
  ld.v_part(s, wave, lane);
  ld.gate_next(t0, w.tok_end);
  ld.g_part(s, wave, lane, 0);
  ld.gate_next(t0 + C, w.tok_end);
  ld.g_part(s, wave, lane, 1);
  barrier_all();
  // With the x loads inside the chunk loop, the initial-state loads must be
  // known drained here, or the compiler's wait insertion would wait for every
  // later load (the x loads included) before their first use in the loop.
  if constexpr (DOT) counters_drained();
  // gates of the first chunk; each later chunk's are prepared at the end of
  // the chunk before it, from the ring slot loaded two chunks ahead
  float gam = 1.f;
  if (t0 < w.tok_end) {
    const float x = s.lgb[0][lane];
    gam = R.gates(lane < w.tok_end - t0 ? x : 0.f, lsum);
  }
  int g_rd = 1, g_ld = 2;  // ring slots of the next chunk's and of the far chunk's gates

  // key rows of this wavefront's 32 keys (js = rh) and of the partner's
  const int jo = 32 * rh, jx = 32 * (1 - rh);
  // score tiles: tile `wave` (with four column groups every wavefront, and
  // tiles 8 and 9 also for wavefronts 4 and 5; with six, wavefronts 0 .. 9),
  // lower triangle of 16x16 tiles, row-major
  // six column groups: the ten tiles on waves 0-3 and 6-11, so that the
  // loading waves 4 and 5 (SIMDs 0 and 1) carry no tile
  const bool has_tile = NCG == 4 || wave < 4 || wave >= 6;
  const int tidx = NCG == 4 || wave < 4 ? wave : wave - 2;
  const int ti1 = tile_ti(has_tile ? tidx : 0), tj1 = tile_tj(has_tile ? tidx : 0);
  const bool two_tiles = NCG == 4 && (wave == 4 || wave == 5);
  const int ti2 = 3, tj2 = wave - 2;

  for (int ci = 0; t0 < w.tok_end; t0 += C, ++ci) {
    const int n = min(C, w.tok_end - t0);
    const int st = ci & 1;
    // chunk ci's tiles are in LDS and every wavefront left chunk ci-1; the
    // output stores of chunk ci-1 (at most two, issued after this wavefront's
    // loads had all completed) may still be in flight. The state pass stores
    // nothing and waits for everything.
    if (SP) {
      barrier_all();
      counters_drained();
    } else if (DOT) {  // two output and two dot-product stores
      barrier_all_but_4();
      counters_drained_but_4();
    } else {
      barrier_all_but_2();
      counters_drained_but_2();
    }

    const uint16_t *sq = s.q[SP ? 0 : st];
    const uint16_t *sk = s.k[st];
    const uint16_t *sv = s.v[st];
    const bool has_next = t0 + C < w.tok_end;
    if (wave < Loader::LW) {  // only the loading wavefronts need descriptors
      ld.next(t0 + C, w.tok_end, st ^ 1);
      ld.k_part(s, wave, lane);
      if (wave == Loader::LW - 1) {
        ld.gate_next(t0 + 2 * C, w.tok_end);
        ld.g_part(s, wave, lane, g_ld);
      }
    }

    // x row pieces matching this chunk's outputs (DOT); they land long before
    // the chunk-end stores, which wait for every load anyway
    u32x2 xv[2] = {u32x2{0u, 0u}, u32x2{0u, 0u}};
    if constexpr (DOT) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int r = 16 * (m ? mi1 : mi0) + ln;
        if (r < n)
          xv[m] = *reinterpret_cast<const u32x2 *>(
              xd + (mem_row(t0 + r) * H + h) * DV + col0 + wcol + 4 * lg4);
      }
    }

    f32x4 own[2];
    if (!SP) {
      // ---- score tile(s) and the state read over this wavefront's half of
      // d_k for all 64 rows, scheduled together:
      // part[mi][r] = sum over d in the half of S[d][wcol + 4 lg4 + r] Q[16 mi + ln][d]
      // With six column groups the tile runs on its own before the state read
      // (the overlapped schedule needs more registers than three wavefronts
      // per SIMD have).
      constexpr bool kOverlapTile = NCG == 4;
      if (!kOverlapTile && has_tile) {
        typename Wv::TileOps t0;
        R.tile_read(t0, sq, sk, ti1, tj1);
        R.tile_store(R.tile_mma(t0), t0, R.tile_mask(ti1, tj1, t0.rq), ti1, tj1);
      }
      typename Wv::TileOps t1;
      if (kOverlapTile && has_tile) R.tile_read(t1, sq, sk, ti1, tj1);
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
      // the last 16 rows of a 48-row half: slot 4 lg4 + r <-> d = drow0 + 32 NKH + 4 lg4 + r
      u32x2 qr[QREM ? 4 : 1];
      if constexpr (QREM) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          qr[mi] = *reinterpret_cast<const u32x2 *>(
              &sq[qk_off<DK>(16 * mi + ln, drow0 + 32 * NKH + 4 * lg4)]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // hi/lo bf16 of the state half (A operand), while the reads are in flight:
      // slot 8 lg4 + r <-> d = drow0 + 32 ks + 4 lg4 + r,
      // slot 8 lg4 + 4 + r <-> d = drow0 + 32 ks + 16 + 4 lg4 + r
      u32x4 sh[NKH], sl[NKH];
#pragma unroll
      for (int ks = 0; ks < NKH; ++ks) {
        uint32_t h[4], l[4];
        split_pk_bf16(S_acc[2 * ks][0], S_acc[2 * ks][1], h[0], l[0]);
        split_pk_bf16(S_acc[2 * ks][2], S_acc[2 * ks][3], h[1], l[1]);
        split_pk_bf16(S_acc[2 * ks + 1][0], S_acc[2 * ks + 1][1], h[2], l[2]);
        split_pk_bf16(S_acc[2 * ks + 1][2], S_acc[2 * ks + 1][3], h[3], l[3]);
        sh[ks] = u32x4{h[0], h[1], h[2], h[3]};
        sl[ks] = u32x4{l[0], l[1], l[2], l[3]};
      }
      u32x2 srh, srl;
      if constexpr (QREM) {
        uint32_t h0, l0, h1, l1;
        split_pk_bf16(S_acc[2 * NKH][0], S_acc[2 * NKH][1], h0, l0);
        split_pk_bf16(S_acc[2 * NKH][2], S_acc[2 * NKH][3], h1, l1);
        srh = u32x2{h0, h1};
        srl = u32x2{l0, l1};
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x4 acc1 = {0.f, 0.f, 0.f, 0.f};
      if (kOverlapTile && has_tile) acc1 = R.tile_mma(t1);
      f32x4 part[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) part[mi] = mfma16(sh[0], qf[0][mi], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) part[mi] = mfma16(sl[0], qf[0][mi], part[mi]);
      __builtin_amdgcn_sched_barrier(0);
      // the tile's mask and P stores overlap the rest of the state read
      if (kOverlapTile && has_tile) R.tile_store(acc1, t1, R.tile_mask(ti1, tj1, t1.rq), ti1, tj1);
#pragma unroll
      for (int ks = 1; ks < NKH; ++ks) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) part[mi] = mfma16(sh[ks], qf[ks][mi], part[mi]);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) part[mi] = mfma16(sl[ks], qf[ks][mi], part[mi]);
      }
      if constexpr (QREM) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) part[mi] = mfma16k16(srh, qr[mi], part[mi]);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) part[mi] = mfma16k16(srl, qr[mi], part[mi]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (two_tiles) {
        typename Wv::TileOps t2;
        R.tile_read(t2, sq, sk, ti2, tj2);
        R.tile_store(R.tile_mma(t2), t2, R.tile_mask(ti2, tj2, t2.rq), ti2, tj2);
      }
      ld.q_part(s, wave, lane);
      // rows of the partner's blocks go through LDS (rh is wave-uniform: no
      // register indexing)
      if (rh) {
        s.xbuf[wave][0][lane] = part[0];
        s.xbuf[wave][1][lane] = part[3];
        own[0] = part[1];
        own[1] = part[2];
      } else {
        s.xbuf[wave][0][lane] = part[1];
        s.xbuf[wave][1][lane] = part[2];
        own[0] = part[0];
        own[1] = part[3];
      }
    }

    // ---- kappa . V for this wavefront's 32 keys (js = rh), hi/lo; the partner
    // does the other 32. V^T fragments: slot 8 lg4 + e <-> key j0 + 8 lg4 + e,
    // column wcol + ln.
    const f32x4 kap0 = *reinterpret_cast<const f32x4 *>(&s.gkap[wave][jo + 8 * lg4]);
    const f32x4 kap1 = *reinterpret_cast<const f32x4 *>(&s.gkap[wave][jo + 8 * lg4 + 4]);
    auto v_frag = [&](int j0) -> u32x4 {
      const int r0 = j0 + 8 * lg4 + (ln >> 2);
      const int c = wcol + 4 * (ln & 3);
      const u32x2 x0 = lds_tr16_nowait(&sv[v_off_sw<SW>(r0, c)]);
      const u32x2 x1 = lds_tr16_nowait(&sv[v_off_sw<SW>(r0 + 4, c)]);
      return u32x4{x0.x, x0.y, x1.x, x1.y};
    };
    u32x4 vf_0 = v_frag(0);   // keys 0..31
    u32x4 vf_1 = v_frag(32);  // keys 32..63
    lds_wait(vf_0, vf_1);
    const u32x4 vf_o = rh ? vf_1 : vf_0;  // this wavefront's 32 keys
    u32x4 kv_h, kv_l;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const uint32_t vw = vf_o[e2];
      const float v0 = __uint_as_float(vw << 16), v1 = __uint_as_float(vw & 0xffff0000u);
      const f32x4 &kk = e2 < 2 ? kap0 : kap1;
      uint32_t hh, ll;
      split_pk_bf16(kk[2 * (e2 & 1)] * v0, kk[2 * (e2 & 1) + 1] * v1, hh, ll);
      kv_h[e2] = hh;
      kv_l[e2] = ll;
    }
    s.kvx[wave][0][lane] = kv_h;
    s.kvx[wave][1][lane] = kv_l;

    // ---- K^T for the state update, read now and used after the barrier
    // (A operand: slot 8 lg4 + e <-> key j0 + 8 lg4 + e, row d = drow0 + 16 t + ln).
    // With six column groups the partner's keys are read after the barrier,
    // once this wavefront's own keys are in (register budget).
    constexpr bool kEarlyKx = NCG == 4;
    u32x4 kt_o[NTH], kt_x[NTH];
    auto kt_read = [&](int j0, int t) -> u32x4 {
      const int c = drow0 + 16 * t + 4 * (ln & 3);
      const int r = j0 + 8 * lg4 + (ln >> 2);
      const u32x2 a0 = lds_tr16_nowait(&sk[qk_off<DK>(r, c)]);
      const u32x2 a1 = lds_tr16_nowait(&sk[qk_off<DK>(r + 4, c)]);
      return u32x4{a0.x, a0.y, a1.x, a1.y};
    };
    if constexpr (kEarlyKx) {
#pragma unroll
      for (int t = 0; t < NTH; ++t) {
        const int c = drow0 + 16 * t + 4 * (ln & 3);
        const int ro = jo + 8 * lg4 + (ln >> 2), rx = jx + 8 * lg4 + (ln >> 2);
        const u32x2 a0 = lds_tr16_nowait(&sk[qk_off<DK>(ro, c)]);
        const u32x2 a1 = lds_tr16_nowait(&sk[qk_off<DK>(ro + 4, c)]);
        const u32x2 b0 = lds_tr16_nowait(&sk[qk_off<DK>(rx, c)]);
        const u32x2 b1 = lds_tr16_nowait(&sk[qk_off<DK>(rx + 4, c)]);
        kt_o[t] = u32x4{a0.x, a0.y, a1.x, a1.y};
        kt_x[t] = u32x4{b0.x, b0.y, b1.x, b1.y};
      }
    } else {
#pragma unroll
      for (int t = 0; t < NTH; ++t) kt_o[t] = kt_read(jo, t);
    }

    ld.v_part(s, wave, lane);
    barrier_lds();  // P, the partial outputs and kappa . V are complete
    static_assert(NTH == 4 || NTH == 3 || NTH == 2, "state tiles per wavefront");
    if constexpr (NTH == 4) {
      lds_after_wait(kt_o[0], kt_o[1], kt_o[2], kt_o[3]);
      lds_after_wait(kt_x[0], kt_x[1], kt_x[2], kt_x[3]);
    } else if constexpr (NTH == 3) {  // six column groups: the partner's keys come later
      static_assert(!kEarlyKx, "three state tiles go with six column groups");
      lds_after_wait(kt_o[0], kt_o[1], kt_o[2]);
    } else {
      lds_after_wait(kt_o[0], kt_o[1], kt_x[0], kt_x[1]);
    }

    // operands of P V and of the rest of the state update
    const u32x4 kx_h = s.kvx[pw][0][lane];
    const u32x4 kx_l = s.kvx[pw][1][lane];
    // P fragments: block mi0 (rows < 32) needs keys 0..31, block mi1 (rows >= 32) all 64
    u32x4 pf_h[3], pf_l[3];
    f32x4 xp[2];
    float lam[2];
    if (!SP) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int mi = m ? mi1 : mi0;
        xp[m] = s.xbuf[pw][m][lane];
        lam[m] = s.glam[wave][16 * mi + ln];
      }
#pragma unroll
      for (int e = 0; e < 3; ++e) {
        const int off = (16 * (e ? mi1 : mi0) + ln) * PP + 32 * (e == 2) + 8 * lg4;
        pf_h[e] = *reinterpret_cast<const u32x4 *>(&s.phi[off]);
        pf_l[e] = *reinterpret_cast<const u32x4 *>(&s.plo[off]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- state advance for this half, S <- gamma S + K_half^T (kappa . V):
    // this wavefront's own 32 keys first (nothing read after the barrier)
#pragma unroll
    for (int t = 0; t < NTH; ++t) S_acc[t] *= gam;
#pragma unroll
    for (int t = 0; t < NTH; ++t) S_acc[t] = mfma16(kt_o[t], kv_h, S_acc[t]);
#pragma unroll
    for (int t = 0; t < NTH; ++t) S_acc[t] = mfma16(kt_o[t], kv_l, S_acc[t]);
    __builtin_amdgcn_sched_barrier(0);

    if (!SP) {
      // own rows: partner's half of the state read, scale by 2^(b2_i), then V^T P^T
#pragma unroll
      for (int m = 0; m < 2; ++m) own[m] = (own[m] + xp[m]) * lam[m];
      own[0] = mfma16(vf_0, pf_h[0], own[0]);
      own[1] = mfma16(vf_0, pf_h[1], own[1]);
      own[0] = mfma16(vf_0, pf_l[0], own[0]);
      own[1] = mfma16(vf_0, pf_l[1], own[1]);
      own[1] = mfma16(vf_1, pf_h[2], own[1]);
      own[1] = mfma16(vf_1, pf_l[2], own[1]);
    }
    // the partner's 32 keys
    if constexpr (!kEarlyKx) {
#pragma unroll
      for (int t = 0; t < NTH; ++t) kt_x[t] = kt_read(jx, t);
      static_assert(kEarlyKx || NTH == 3, "late partner keys: three state tiles");
      lds_wait(kt_x[0], kt_x[1], kt_x[2]);
    }
#pragma unroll
    for (int t = 0; t < NTH; ++t) S_acc[t] = mfma16(kt_x[t], kx_h, S_acc[t]);
#pragma unroll
    for (int t = 0; t < NTH; ++t) S_acc[t] = mfma16(kt_x[t], kx_l, S_acc[t]);

    if (has_next) {
      const float x = s.lgb[g_rd][lane];
      gam = R.gates(lane < w.tok_end - t0 - C ? x : 0.f, lsum);
    }
    if (!SP) store_out(t0, n, own, xv);
    g_rd = g_rd == 2 ? 0 : g_rd + 1;
    g_ld = g_ld == 2 ? 0 : g_ld + 1;
  }

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

template <int DK, int NCG, typename Tout, bool SP, bool REV = false, bool DOT = false>
static hipError_t launch_w8_t(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *g, const float *S0, float *S_T, void *o,
                              const FwdDims &d, const WorkItem *items, const int *n_items,
                              int grid_items, float *slots, float *slot_gamma,
                              hipStream_t stream) {
  const long pairs = (long)grid_items * d.H;
  const long blocks = pairs * (d.dv / (16 * NCG));
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_bf16_w8_kernel<DK, NCG, Tout, SP, REV, DOT>), dim3(blocks),
                     dim3(128 * NCG), 0, stream, q, k, v, g, S0, S_T, static_cast<Tout *>(o),
                     items, n_items, slots, slot_gamma, d.T, d.H, d.gts, d.dv, (int)pairs,
                     d.dot_x, d.dot_part, d.dot_stride, d.hg, static_cast<Tout *>(d.o2));
  return hipGetLastError();
}

template <int DK, int NCG>
static hipError_t launch_w8_d(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *g, const float *S0, float *S_T, void *o, bool out_bf16,
                              const FwdDims &d, const WorkItem *items, const int *n_items,
                              int grid_items, float *slots, float *slot_gamma, bool state_pass,
                              hipStream_t stream) {
  if constexpr (NCG == 4) {  // the backward's runs: fp32 outputs, optionally reversed / dots
    if (d.rev || d.dot_x) {
      if (state_pass) {
        if (d.rev)
          return launch_w8_t<DK, NCG, float, true, true>(q, k, v, g, S0, S_T, o, d, items,
                                                         n_items, grid_items, slots, slot_gamma,
                                                         stream);
      } else {
        if (out_bf16) return hipErrorInvalidValue;
        if (d.rev && d.dot_x)
          return launch_w8_t<DK, NCG, float, false, true, true>(q, k, v, g, S0, S_T, o, d, items,
                                                                n_items, grid_items, slots,
                                                                slot_gamma, stream);
        if (d.rev)
          return launch_w8_t<DK, NCG, float, false, true>(q, k, v, g, S0, S_T, o, d, items,
                                                          n_items, grid_items, slots, slot_gamma,
                                                          stream);
        return launch_w8_t<DK, NCG, float, false, false, true>(q, k, v, g, S0, S_T, o, d, items,
                                                               n_items, grid_items, slots,
                                                               slot_gamma, stream);
      }
    }
  } else {  // 96 x 192 heads: the backward's dv run (reversed, fp32 output, no dots)
    if (d.dot_x) return hipErrorInvalidValue;
    if (d.rev) {
      if (state_pass)
        return launch_w8_t<DK, NCG, float, true, true>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                                       grid_items, slots, slot_gamma, stream);
      if (out_bf16) return hipErrorInvalidValue;
      return launch_w8_t<DK, NCG, float, false, true>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                                      grid_items, slots, slot_gamma, stream);
    }
  }
  if (state_pass)
    return launch_w8_t<DK, NCG, float, true>(q, k, v, g, S0, S_T, o, d, items, n_items, grid_items,
                                        slots, slot_gamma, stream);
  if (out_bf16)
    return launch_w8_t<DK, NCG, uint16_t, false>(q, k, v, g, S0, S_T, o, d, items, n_items,
                                            grid_items, slots, slot_gamma, stream);
  return launch_w8_t<DK, NCG, float, false>(q, k, v, g, S0, S_T, o, d, items, n_items, grid_items,
                                       slots, slot_gamma, stream);
}

hipError_t launch_chunk_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const float *g, const float *S0, float *S_T, void *o, bool out_bf16,
                             const FwdDims &d, const WorkItem *items, const int *n_items,
                             int grid_items, float *slots, float *slot_gamma, bool state_pass,
                             hipStream_t stream) {
  if (d.C != kW8C) return hipErrorInvalidValue;  // the planner runs bf16 inputs at chunk 64
  if (d.hg != 1 && (d.dot_x || d.H % d.hg || !d.o2)) return hipErrorInvalidValue;
  // 128-dim keys (forward and the backward's runs, and their state passes):
  // the wavefront-specialised kernels
  if (!state_pass && d.dk == 128 && d.dv % 64 == 0 && d.hg == 1 &&
      !((d.rev || d.dot_x) && (out_bf16 || d.gts == 0)))
    return launch_chunk_bf16_ws(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                                slots, stream);
  if (state_pass && d.dk == 128 && d.dv % 64 == 0 && d.hg == 1)
    return launch_chunk_bf16_ws_state(k, v, g, d, items, n_items, grid_items, slots, slot_gamma,
                                      stream);
  if (d.dk == 96)  // 96 x 192 heads: two slices of six column groups
    return launch_w8_d<96, 6>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                              slots, slot_gamma, state_pass, stream);
  if (d.dk == 128)
    return launch_w8_d<128, 4>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items,
                               slots, slot_gamma, state_pass, stream);
  return launch_w8_d<64, 4>(q, k, v, g, S0, S_T, o, out_bf16, d, items, n_items, grid_items, slots,
                         slot_gamma, state_pass, stream);
}

}  // namespace gla
