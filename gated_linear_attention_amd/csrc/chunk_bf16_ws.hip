// Chunked GLA forward for bf16 inputs with 128-dim keys on the CDNA4 matrix
// cores: 64-token chunks, eight wavefronts per workgroup in two roles.
//
// Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), "Challenge 1":
// a chunk's output is the query's read of the running state plus
// decay-masked attention within the chunk, and only the state carries from
// chunk to chunk. With b_i the in-chunk inclusive cumulative log-gate:
//
//   O = diag(e^{b}) Q S + ((Q K^T) .* D) V,   D_ij = e^{b_i - b_j} (j <= i)
//   S <- e^{b_last} S + K^T (e^{b_last - b} . V)
//
// Only the two state terms are sequential from chunk to chunk; the
// attention term of a chunk needs nothing but that chunk's tiles. So the
// wavefronts split by that line, one of each kind per SIMD:
//
//   * state wavefronts 0..3 each hold 16 columns of the fp32 state slice over
//     all 128 key dimensions in matrix-core accumulators and, per chunk, form
//     the state read e^{b} Q S for those columns, advance the state, and
//     finish and store the previous chunk's outputs for those columns;
//   * intra wavefronts 4..7 each own one 16-query row block r of the chunk:
//     they compute its r + 1 score tiles K Q^T, apply the decay mask, keep P
//     in registers (as bf16 hi/lo pairs), multiply it into V for all 64
//     columns and hand P V on through LDS; they also copy the tiles
//     HBM -> registers -> LDS, two chunks ahead, and one of them prepares the
//     next chunk's decay arrays.
//
// The two roles meet at one workgroup barrier per step: in step n the state
// wavefronts read the state against chunk n and advance it, and store
// O = e^{b} (Q S) + P V of chunk n-1 from the attention term that step n-1
// left in LDS; the intra wavefronts form chunk n's attention term. P never
// goes through LDS, no partial sums over key dimensions are exchanged, and
// the state chain of a chunk is one wavefront's dependency chain with no
// barrier inside it. Each role's body is compiled on its own (the intra one
// once per row block), so neither holds the other's registers.
//
// Operands and accuracy are those of the eight-wavefront kernel
// (chunk_bf16_w8.hip): tiles swizzled in LDS and read with 16-byte and
// transposing (ds_read_b64_tr_b16) reads; every value rounded on its way into
// a matrix-core product (P, the state, kappa . V) split into bf16 hi and lo
// parts, both multiplied.
#include "bf16_blocks.h"
#include "tile_loader.h"

namespace gla {

namespace {

constexpr int kWsDK = 128;  // key dimensions
constexpr int kWsSW = 64;   // state columns per workgroup slice
constexpr int kWsXP = 68;   // row pitch (floats) of the hand-over: rows 16 B apart in banks

// One chunk's decay arrays (log2 units), prepared one chunk ahead.
struct alignas(16) WsGates {
  float b2[kW8C];   // in-chunk inclusive prefix sums of the log-gates
  float lam[kW8C];  // 2^(b2_i), 0 from the chunk's first reset on
  float kap[kW8C];  // 2^(b2_last - b2_j), 0 before the chunk's last reset
  int rs[kW8C];     // last reset at or before position i (-1: none)
  float gam;        // 2^(b2_last), 0 if the chunk holds a reset
  float pad[3];
};

struct WsLds {
  uint16_t q[2][kW8C * kWsDK];
  uint16_t k[2][kW8C * kWsDK];
  uint16_t v[2][kW8C * kWsSW];
  float y[2][kW8C * kWsXP];  // attention term P V of a chunk, [token][column]
  float lgb[3][kW8C];        // log-gates of the chunks one and two ahead
  WsGates g[2];
};

// LLVM's raw buffer loads into registers (offsets at or past the descriptor's
// range read as 0); the last argument is the cache policy (kNonTemporal: nt).
constexpr int kNonTemporal = 2;
__device__ i32x4 raw_buffer_load_b128(i32x4 rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.v4i32");
__device__ float raw_buffer_load_f32(i32x4 rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.f32");

// HBM -> LDS copies of the intra wavefronts, staged in registers: a chunk is
// loaded in one step and written to LDS at the start of the next, so a load
// has a whole step to land and the tiles need only two LDS stages. Intra
// wavefront iw loads K and Q 1 KB blocks 4 iw .. 4 iw + 3 (4 rows of 256 B
// each) and V blocks 2 iw, 2 iw + 1 (8 rows of 128 B), 16 bytes a lane with
// the 16-byte chunks swizzled as qk_off / v_off place them (the global side
// reads the swizzled chunk, the LDS side is linear); the last one also loads
// the log-gates, three chunks ahead. Rows past the end of the run lie past
// the descriptor's range and read as zeros.
//
// REV (time-reversed run, the backward's adjoint recurrence): logical token t
// of a sequence [sb, se) is memory row sb + se - 1 - t, so a chunk's rows are
// read bottom-up into the same LDS layout, and the gate at logical position
// u = t - sb is the log-gate of memory row se - u (u >= 1; 0 at u = 0).
//
// QL = false (the state pass): K and V only.
template <bool REV, bool QL = true>
struct WsStager {
  static constexpr int C = kW8C, DK = kWsDK, SW = kWsSW;
  static constexpr int kFar = 0x7fff0000;  // an offset past any descriptor range
  const uint16_t *qp, *kp, *vp;  // first row (this head / slice) of the next chunk to load
  const float *gp;               // first gate of the next gate chunk to load
  size_t qk_step, v_step, g_step;
  uint32_t qk_row, v_row, g_row;  // bytes per token
  u32x4 kq[8], vv[2];             // staged K (0..3) and Q (4..7) blocks, V blocks
  float gx;                       // staged log-gate
  bool active, g_active;
  // REV: head / slice bases, sb + se and the sequence start
  const uint16_t *qh, *kh, *vh;
  const float *gh;
  int se_sum, seq_b;

  __device__ __forceinline__ void init(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                       const float *lg, int t0, int H, int gts, int h, int DV,
                                       int col0, int sb, int se) {
    if constexpr (REV) {
      qh = q + (size_t)h * DK;
      kh = k + (size_t)h * DK;
      vh = v + (size_t)h * DV + col0;
      gh = lg + h;
      se_sum = sb + se;
      seq_b = sb;
    }
    const size_t tok0 = (size_t)t0 * H + h;
    qp = q + tok0 * DK;
    kp = k + tok0 * DK;
    vp = v + tok0 * DV + col0;
    gp = lg + (size_t)t0 * gts + h;
    qk_step = (size_t)C * H * DK;
    v_step = (size_t)C * H * DV;
    g_step = (size_t)C * gts;
    qk_row = (uint32_t)H * DK * 2;
    v_row = (uint32_t)H * DV * 2;
    g_row = (uint32_t)gts * 4;
  }
  // Load the chunk that starts at t0 (the one after the previous call's).
  __device__ __forceinline__ void load(int t0, int tok_end, int iw, int lane) {
    active = t0 < tok_end;
    if (!active) return;
    const uint32_t last = (uint32_t)(min(C, tok_end - t0) - 1);
    const int n_ld = (int)last + 1;
    if constexpr (REV) {  // lowest memory row of the chunk: sb + se - t0 - n
      const size_t lo = (size_t)(se_sum - t0 - n_ld);
      qp = qh + lo * (qk_row / 2);
      kp = kh + lo * (qk_row / 2);
      vp = vh + lo * (v_row / 2);
    }
    const i32x4 rk = make_rsrc(kp, last * qk_row + DK * 2);
    const i32x4 rq = QL ? make_rsrc(qp, last * qk_row + DK * 2) : rk;
    const i32x4 rv = make_rsrc(vp, last * v_row + SW * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (4 * iw + i) * 4 + lane / 16;
      int vo = (REV ? n_ld - 1 - row : row) * qk_row + (((lane % 16) ^ (row & 15)) << 4);
      if (REV && row >= n_ld) vo = kFar;
      kq[i] = __builtin_bit_cast(u32x4, raw_buffer_load_b128(rk, vo, 0, 0));
      if constexpr (QL) kq[4 + i] = __builtin_bit_cast(u32x4, raw_buffer_load_b128(rq, vo, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (2 * iw + i) * 8 + lane / 8;
      int vo = (REV ? n_ld - 1 - r : r) * v_row + (((lane % 8) ^ (r & 7)) << 4);
      if (REV && r >= n_ld) vo = kFar;
      // V is read by this workgroup alone: a non-temporal load (cache policy nt)
      vv[i] = __builtin_bit_cast(u32x4, raw_buffer_load_b128(rv, vo, 0, kNonTemporal));
    }
    qp += qk_step;
    kp += qk_step;
    vp += v_step;
  }
  // Write the staged chunk into stage st.
  template <typename L>
  __device__ __forceinline__ void commit(L &s, int st, int iw, int lane) {
    if (!active) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4 *>(&s.k[st][(4 * iw + i) * 512 + 8 * lane]) = kq[i];
      if constexpr (QL)
        *reinterpret_cast<u32x4 *>(&s.q[st][(4 * iw + i) * 512 + 8 * lane]) = kq[4 + i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4 *>(&s.v[st][(2 * iw + i) * 512 + 8 * lane]) = vv[i];
  }
  // The log-gates of the chunk at t0 (a per-token stream: lanes past the end
  // read 0; a fixed decay, stride 0: every lane reads the head's value).
  __device__ __forceinline__ void gate_load(int t0, int tok_end, int lane) {
    g_active = t0 < tok_end;
    if (!g_active) return;
    const uint32_t last = (uint32_t)(min(C, tok_end - t0) - 1);
    if constexpr (REV) {  // rows se - u for u = t0 - sb + n - 1 .. t0 - sb; u = 0 is out of range
      const int n_g = (int)last + 1;
      const i32x4 rg = make_rsrc(gh + (size_t)(se_sum - t0 - n_g + 1) * (g_row / 4),
                                 last * g_row + (t0 == seq_b ? 0 : 4));
      gx = raw_buffer_load_f32(rg, lane < n_g ? (n_g - 1 - lane) * g_row : kFar, 0, 0);
      return;
    }
    gx = raw_buffer_load_f32(make_rsrc(gp, last * g_row + 4), lane * g_row, 0, 0);
    gp += g_step;
  }
  template <typename L>
  __device__ __forceinline__ void gate_commit(L &s, int slot, int lane) {
    if (g_active) s.lgb[slot][lane] = gx;
  }
};

// The decay arrays of a chunk from its log-gates (x = this lane's, 0 past the
// end of the run): a reset gate enters the prefix sums as 0 and cuts every
// product of gates that spans it. Returns the chunk's total log-decay (-inf if
// it holds a reset).
__device__ __forceinline__ float ws_gates(WsGates &g, float x, int lane) {
  const bool rst = is_reset(x);
  const uint64_t rm = __builtin_amdgcn_ballot_w64(rst);
  const float incl = wave_inclusive_scan(rst ? 0.f : x);
  const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
  const float b2last = total * kLog2e;
  const float b2 = incl * kLog2e;
  const int ri = last_set_upto(rm, lane), rl = last_set(rm);
  g.b2[lane] = b2;
  g.rs[lane] = ri;
  g.lam[lane] = ri < 0 ? fast_exp2(b2) : 0.f;
  g.kap[lane] = lane < rl ? 0.f : fast_exp2(b2last - b2);
  if (lane == 0) g.gam = rl < 0 ? fast_exp2(b2last) : 0.f;
  return rl < 0 ? total : -__builtin_huge_valf();
}

// The attention term of one chunk for query row block R (rows 16 R .. 16 R +
// 15): score tiles A^T = K Q^T (rows: keys 16 tj + 4 lg4 + r, columns:
// queries 16 R + ln), decay-masked into bf16 hi/lo P held in registers, then
// V^T P^T for all 64 columns, written to y[token][column] in 16-byte row
// pieces. B = P^T for keys 32 kb .. 32 kb + 31: slot e < 4 <-> key 32 kb +
// 4 lg4 + e (tile 2 kb), e >= 4 <-> key 32 kb + 16 + 4 lg4 + e - 4 (tile
// 2 kb + 1, zero above the diagonal); A = V^T with the same key slots.
template <int R>
__device__ __forceinline__ void ws_intra(const uint16_t *sq, const uint16_t *sk,
                                         const uint16_t *sv, const WsGates &G, float *y, int ln,
                                         int lg4) {
  constexpr int DK = kWsDK, XP = kWsXP;
  constexpr int NT = R + 1;         // score tiles of the row block
  constexpr int NKB = (R + 2) / 2;  // 32-key steps of P V
  const int qrow = 16 * R + ln;
  u32x4 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qb[ks] = *reinterpret_cast<const u32x4 *>(&sq[qk_off<DK>(qrow, 32 * ks + 8 * lg4)]);
  const float b2q = G.b2[qrow];
  const int rq = G.rs[qrow];
  uint32_t ph[2 * NKB][2], pl[2 * NKB][2];
#pragma unroll
  for (int tj = 0; tj < 2 * NKB; ++tj) ph[tj][0] = ph[tj][1] = pl[tj][0] = pl[tj][1] = 0u;
#pragma unroll
  for (int tj = 0; tj < NT; ++tj) {
    u32x4 a[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      a[ks] = *reinterpret_cast<const u32x4 *>(&sk[qk_off<DK>(16 * tj + ln, 32 * ks + 8 * lg4)]);
    const f32x4 g4 = *reinterpret_cast<const f32x4 *>(&G.b2[16 * tj + 4 * lg4]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma16(a[ks], qb[ks], acc);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * tj + 4 * lg4 + r;
      const bool keep = (tj < R || j <= qrow) && j >= rq;
      p[r] = acc[r] * fast_exp2(b2q - g4[r] + (keep ? 0.f : -__builtin_huge_valf()));
    }
    split_pk_bf16(p[0], p[1], ph[tj][0], pl[tj][0]);
    split_pk_bf16(p[2], p[3], ph[tj][1], pl[tj][1]);
  }
  f32x4 oi[4] = {};
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const u32x4 bh = {ph[2 * kb][0], ph[2 * kb][1], ph[2 * kb + 1][0], ph[2 * kb + 1][1]};
    const u32x4 bl = {pl[2 * kb][0], pl[2 * kb][1], pl[2 * kb + 1][0], pl[2 * kb + 1][1]};
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int cc = 16 * ct + 4 * (ln & 3);
      const u32x2 x0 = lds_tr16(&sv[v_off(32 * kb + 4 * lg4 + (ln >> 2), cc)]);
      const u32x2 x1 = lds_tr16(&sv[v_off(32 * kb + 16 + 4 * lg4 + (ln >> 2), cc)]);
      const u32x4 va = u32x4{x0.x, x0.y, x1.x, x1.y};
      oi[ct] = mfma16(va, bh, oi[ct]);
      oi[ct] = mfma16(va, bl, oi[ct]);
    }
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
    *reinterpret_cast<f32x4 *>(&y[qrow * XP + 16 * ct + 4 * lg4]) = oi[ct];
}

}  // namespace

// REV: the time-reversed run (see WsStager). DOT: also the row dot products
// of the outputs with x (a bf16 tensor of the outputs' shape): each state
// wavefront sums o * x over its 16 columns per row and writes
// part[((slice * 4 + column group) * H + h) * part_stride + token].
template <typename Tout, bool REV, bool DOT>
__global__ __launch_bounds__(512) void chunk_bf16_ws_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ lg, const float *__restrict__ S0,
    float *__restrict__ ST, Tout *__restrict__ o, const WorkItem *__restrict__ items,
    const int *__restrict__ n_items, const float *__restrict__ slots, int T, int H, int gts,
    int DV, int n_pairs, const uint16_t *__restrict__ xd, float *__restrict__ dpart,
    long part_stride) {
  constexpr int C = kW8C, DK = kWsDK, SW = kWsSW, XP = kWsXP;
  __shared__ WsLds s;

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
  if (items && it >= *n_items) return;
  const WorkItem w = bf_item_for(items, it, T);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int ln = lane % 16, lg4 = lane / 16;
  const bool state_wave = wave < 4;
  const int c = wave & 3;  // state: column group of 16; intra: row block of 16 queries
  const int iw = wave - 4; // index among the intra (loading) wavefronts
  const int col0 = slice * SW;
  const size_t dkdv = (size_t)DK * DV;
  // the state chain is the longer one: let the SIMD arbiter prefer it
  if (state_wave) __builtin_amdgcn_s_setprio(2);

  // State columns of a state wavefront, accumulator layout:
  // S_acc[t][r] = S[16 t + 4 lg4 + r][col0 + 16 c + ln].
  f32x4 S_acc[8];
  if (state_wave) {
    const float *sin = nullptr;
    if (w.state_in >= 0) sin = slots + ((size_t)w.state_in * H + h) * dkdv;
    else if (S0) sin = S0 + ((size_t)w.seq * H + h) * dkdv;
    if (sin) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S_acc[t][r] = sin[(size_t)(16 * t + 4 * lg4 + r) * DV + col0 + 16 * c + ln];
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) S_acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  const int t0 = w.tok_begin;
  const int NC = (w.tok_end - t0 + C - 1) / C;  // chunks of this run
  // BAL: wavefront 4 (row block 0, the lightest attention term) also copies
  // the tile share of wavefront 7 (row block 3, the heaviest), so that the
  // SIMDs' loads even out; the forward only (the backward's reversed and
  // dot-product runs measured slower with it)
  constexpr bool BAL = !REV && !DOT;
  WsStager<REV> sg, sg2;
  if (!state_wave) {
    // chunk 0 and the gates of chunks 0, 1 straight into LDS; chunk 1 and the
    // gates of chunk 2 staged for the first step
    sg.init(q, k, v, lg, t0, H, gts, h, DV, col0, w.seq_begin, w.seq_end);
    if (!BAL || iw != 3) {
      sg.load(t0, w.tok_end, iw, lane);
      sg.commit(s, 0, iw, lane);
      sg.load(t0 + C, w.tok_end, iw, lane);
    }
    if (BAL && iw == 0) {
      sg2.init(q, k, v, lg, t0, H, gts, h, DV, col0, w.seq_begin, w.seq_end);
      sg2.load(t0, w.tok_end, 3, lane);
      sg2.commit(s, 0, 3, lane);
      sg2.load(t0 + C, w.tok_end, 3, lane);
    }
    if (iw == 3) {
      sg.gate_load(t0, w.tok_end, lane);
      sg.gate_commit(s, 0, lane);
      sg.gate_load(t0 + C, w.tok_end, lane);
      sg.gate_commit(s, 1, lane);
      sg.gate_load(t0 + 2 * C, w.tok_end, lane);
    }
  }
  barrier_lds();
  if (wave == 4 && NC > 0) {
    const float x = s.lgb[0][lane];
    ws_gates(s.g[0], lane < w.tok_end - t0 ? x : 0.f, lane);
  }
  barrier_lds();

  // memory row of logical token t
  auto mem_row = [&](int t) -> size_t {
    return (size_t)(REV ? w.seq_begin + w.seq_end - 1 - t : t);
  };
  if (state_wave) {
    f32x4 qs_prev[4] = {};  // e^{b} Q S of the previous chunk, this wavefront's columns
    for (int ci = 0; ci <= NC; ++ci) {
      const int st = ci & 1;
      const bool cur = ci < NC;
      const WsGates &G = s.g[st];
      const uint16_t *sq = s.q[st];
      const uint16_t *sk = s.k[st];
      const uint16_t *sv = s.v[st];
      f32x4 qs_cur[4];
      // x row pieces matching chunk ci - 1's outputs (DOT), loaded now so that
      // they land while the state is read and advanced
      u32x2 xv[4] = {};
      if constexpr (DOT) {
        if (ci > 0) {
          const int tp = t0 + (ci - 1) * C;
          const int np = min(C, w.tok_end - tp);
#pragma unroll
          for (int m = 0; m < 4; ++m)
            if (16 * m + ln < np)
              xv[m] = *reinterpret_cast<const u32x2 *>(
                  xd + (mem_row(tp + 16 * m + ln) * H + h) * DV + col0 + 16 * c + 4 * lg4);
        }
      }
      if (cur) {
        // ---- state read for this wavefront's 16 columns, all 64 rows:
        // part[m][r] = sum_d S[d][16 c + 4 lg4 + r] Q[16 m + ln][d]. A = S^T
        // (hi, lo) from two accumulator tiles; slot 8 lg4 + r <-> d = 32 ks +
        // 4 lg4 + r, slot 8 lg4 + 4 + r <-> d = 32 ks + 16 + 4 lg4 + r.
        u32x4 qf[4][4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int r = 16 * m + ln;
            const u32x2 qa = *reinterpret_cast<const u32x2 *>(&sq[qk_off<DK>(r, 32 * ks + 4 * lg4)]);
            const u32x2 qb =
                *reinterpret_cast<const u32x2 *>(&sq[qk_off<DK>(r, 32 * ks + 16 + 4 * lg4)]);
            qf[ks][m] = u32x4{qa.x, qa.y, qb.x, qb.y};
          }
        u32x4 sh[4], sl[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          uint32_t hh[4], ll[4];
          split_pk_bf16(S_acc[2 * ks][0], S_acc[2 * ks][1], hh[0], ll[0]);
          split_pk_bf16(S_acc[2 * ks][2], S_acc[2 * ks][3], hh[1], ll[1]);
          split_pk_bf16(S_acc[2 * ks + 1][0], S_acc[2 * ks + 1][1], hh[2], ll[2]);
          split_pk_bf16(S_acc[2 * ks + 1][2], S_acc[2 * ks + 1][3], hh[3], ll[3]);
          sh[ks] = u32x4{hh[0], hh[1], hh[2], hh[3]};
          sl[ks] = u32x4{ll[0], ll[1], ll[2], ll[3]};
        }
        f32x4 part[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) part[m] = mfma16(sh[0], qf[0][m], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int m = 0; m < 4; ++m) part[m] = mfma16(sl[0], qf[0][m], part[m]);
#pragma unroll
        for (int ks = 1; ks < 4; ++ks) {
#pragma unroll
          for (int m = 0; m < 4; ++m) part[m] = mfma16(sh[ks], qf[ks][m], part[m]);
#pragma unroll
          for (int m = 0; m < 4; ++m) part[m] = mfma16(sl[ks], qf[ks][m], part[m]);
        }
        // e^{b_i} of each row, and the state read kept for the next step
#pragma unroll
        for (int m = 0; m < 4; ++m) qs_cur[m] = part[m] * G.lam[16 * m + ln];

        // ---- kappa . V for this wavefront's columns (B operand of the update:
        // slot 8 lg4 + e <-> key 32 kb + 8 lg4 + e, column 16 c + ln), hi/lo
        u32x4 kv_h[2], kv_l[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int r0 = 32 * kb + 8 * lg4 + (ln >> 2);
          const int cc = 16 * c + 4 * (ln & 3);
          const u32x2 x0 = lds_tr16(&sv[v_off(r0, cc)]);
          const u32x2 x1 = lds_tr16(&sv[v_off(r0 + 4, cc)]);
          const u32x4 vf = u32x4{x0.x, x0.y, x1.x, x1.y};
          const f32x4 kap0 = *reinterpret_cast<const f32x4 *>(&G.kap[32 * kb + 8 * lg4]);
          const f32x4 kap1 = *reinterpret_cast<const f32x4 *>(&G.kap[32 * kb + 8 * lg4 + 4]);
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const uint32_t vw = vf[e2];
            const float v0 = __uint_as_float(vw << 16), v1 = __uint_as_float(vw & 0xffff0000u);
            const f32x4 &kk = e2 < 2 ? kap0 : kap1;
            uint32_t hh, ll;
            split_pk_bf16(kk[2 * (e2 & 1)] * v0, kk[2 * (e2 & 1) + 1] * v1, hh, ll);
            kv_h[kb][e2] = hh;
            kv_l[kb][e2] = ll;
          }
        }
        // ---- S <- gamma S + K^T (kappa . V); A = K^T: slot 8 lg4 + e <->
        // key 32 kb + 8 lg4 + e, row d = 16 t + ln. All operands first, then
        // the 32 products ordered so that each accumulator's four are 8 apart.
        u32x4 kt[8][2];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const int r = 32 * kb + 8 * lg4 + (ln >> 2);
            const int cc = 16 * t + 4 * (ln & 3);
            const u32x2 a0 = lds_tr16(&sk[qk_off<DK>(r, cc)]);
            const u32x2 a1 = lds_tr16(&sk[qk_off<DK>(r + 4, cc)]);
            kt[t][kb] = u32x4{a0.x, a0.y, a1.x, a1.y};
          }
        const float gam = G.gam;
#pragma unroll
        for (int t = 0; t < 8; ++t) S_acc[t] *= gam;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int t = 0; t < 8; ++t) S_acc[t] = mfma16(kt[t][kb], kv_h[kb], S_acc[t]);
#pragma unroll
          for (int t = 0; t < 8; ++t) S_acc[t] = mfma16(kt[t][kb], kv_l[kb], S_acc[t]);
        }
      }
      // ---- finish chunk ci - 1 for this wavefront's columns: O = e^{b} Q S
      // + P V, 16-byte row pieces (rows 16 m + ln, columns 16 c + 4 lg4 ..)
      if (ci > 0) {
        const int tp = t0 + (ci - 1) * C;
        const int np = min(C, w.tok_end - tp);
        Tout *ob = o + (size_t)h * DV + col0 + 16 * c + 4 * lg4;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f32x4 pv =
              *reinterpret_cast<const f32x4 *>(&s.y[st ^ 1][(16 * m + ln) * XP + 16 * c + 4 * lg4]);
          const f32x4 out = qs_prev[m] + pv;
          const size_t mr = mem_row(tp + 16 * m + ln);
          if (16 * m + ln < np) store4_from_f32(ob + mr * H * DV, out);
          if constexpr (DOT) {
            const u32x2 xw = xv[m];
            float d = out[0] * __uint_as_float(xw.x << 16) +
                      out[1] * __uint_as_float(xw.x & 0xffff0000u) +
                      out[2] * __uint_as_float(xw.y << 16) +
                      out[3] * __uint_as_float(xw.y & 0xffff0000u);
            // the sum over the row's four lane groups: swapping a value with
            // itself across 16-lane rows (then 32-lane halves) and adding the
            // two results gives d[l] + d[l ^ 16] (then + d[l ^ 32]) everywhere
            const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(d),
                                                              __float_as_uint(d), false, false);
            d = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
            const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(d),
                                                              __float_as_uint(d), false, false);
            d = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
            if (lg4 == 0 && 16 * m + ln < np)
              dpart[((size_t)(slice * 4 + c) * H + h) * part_stride + mr] = d;
          }
        }
      }
      if (cur) {
#pragma unroll
        for (int m = 0; m < 4; ++m) qs_prev[m] = qs_cur[m];
      }
      // the attention term of chunk ci is in LDS; the next chunk's tiles and
      // decay arrays are ready (the output stores stay in flight)
      barrier_lds();
    }
    if (w.state_out == -1 && ST) {
      float *sout = ST + ((size_t)w.seq * H + h) * dkdv;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sout[(size_t)(16 * t + 4 * lg4 + r) * DV + col0 + 16 * c + ln] = S_acc[t][r];
    }
    return;
  }

  // intra wavefronts
  for (int ci = 0; ci <= NC; ++ci) {
    const int tc = t0 + ci * C;  // first token of chunk ci
    const int st = ci & 1;
    const bool cur = ci < NC;
    const WsGates &G = s.g[st];
    const uint16_t *sq = s.q[st];
    const uint16_t *sk = s.k[st];
    const uint16_t *sv = s.v[st];
    // ---- chunk ci + 1 (loaded last step) into the other stage, the gates
    // of chunk ci + 2 into the ring; then load chunk ci + 2 and the gates of
    // chunk ci + 3
    if (!BAL || iw != 3) sg.commit(s, st ^ 1, iw, lane);
    if (BAL && iw == 0) sg2.commit(s, st ^ 1, 3, lane);
    if (iw == 3) sg.gate_commit(s, (ci + 2) % 3, lane);
    if (!BAL || iw != 3) sg.load(tc + 2 * C, w.tok_end, iw, lane);
    if (BAL && iw == 0) sg2.load(tc + 2 * C, w.tok_end, 3, lane);
    if (iw == 3) sg.gate_load(tc + 3 * C, w.tok_end, lane);

    if (cur) {
      switch (c) {  // wave-uniform: one fully unrolled body per row block
        case 0: ws_intra<0>(sq, sk, sv, G, s.y[st], ln, lg4); break;
        case 1: ws_intra<1>(sq, sk, sv, G, s.y[st], ln, lg4); break;
        case 2: ws_intra<2>(sq, sk, sv, G, s.y[st], ln, lg4); break;
        default: ws_intra<3>(sq, sk, sv, G, s.y[st], ln, lg4); break;
      }
    }

    // ---- the decay arrays of chunk ci + 1 (its gates were written last step)
    if (wave == 4 && ci + 1 < NC) {
      const float x = s.lgb[(ci + 1) % 3][lane];
      ws_gates(s.g[st ^ 1], lane < w.tok_end - tc - C ? x : 0.f, lane);
    }
    // chunk ci's attention term, chunk ci + 1's tiles and decay arrays are in
    // LDS (this wavefront's staged loads stay in flight)
    barrier_lds();
  }
}

// The state pass of a split sequence on the same layout: each work item (a
// piece of a segment) runs the state recurrence from zero, S <- e^{b_last} S +
// K^T (kappa . V) chunk by chunk, and leaves its final state in its slot and
// its total log-decay (-inf if it holds a reset) beside it, for the combine to
// chain. No queries, no outputs: the four state wavefronts only advance the
// state; the four others copy K and V two chunks ahead and prepare the decay
// arrays. Without Q, the attention term and the hand-over, a workgroup needs
// 50 KB of LDS and at most 128 VGPRs a lane, so two run on a CU.
struct WsSpLds {
  uint16_t k[2][kW8C * kWsDK];
  uint16_t v[2][kW8C * kWsSW];
  float lgb[3][kW8C];
  WsGates g[2];
};

template <bool REV>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void
chunk_bf16_ws_state_kernel(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                           const float *__restrict__ lg, const WorkItem *__restrict__ items,
                           const int *__restrict__ n_items, float *__restrict__ slots,
                           float *__restrict__ slot_gamma, int T, int H, int gts, int DV,
                           int n_pairs) {
  constexpr int C = kW8C, DK = kWsDK, SW = kWsSW;
  __shared__ WsSpLds s;

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
  if (it >= *n_items) return;
  const WorkItem w = items[it];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int ln = lane % 16, lg4 = lane / 16;
  const bool state_wave = wave < 4;
  const int c = wave & 3;   // state: column group of 16
  const int iw = wave - 4;  // index among the copying wavefronts
  const int col0 = slice * SW;
  const int t0 = w.tok_begin;
  const int NC = (w.tok_end - t0 + C - 1) / C;

  WsStager<REV, false> sg;
  float lsum = 0.f;  // wavefront 4: the item's total log-decay
  if (!state_wave) {
    // (no queries: k stands in for the unused q pointer)
    sg.init(k, k, v, lg, t0, H, gts, h, DV, col0, w.seq_begin, w.seq_end);
    sg.load(t0, w.tok_end, iw, lane);
    sg.commit(s, 0, iw, lane);
    sg.load(t0 + C, w.tok_end, iw, lane);
    if (iw == 3) {
      sg.gate_load(t0, w.tok_end, lane);
      sg.gate_commit(s, 0, lane);
      sg.gate_load(t0 + C, w.tok_end, lane);
      sg.gate_commit(s, 1, lane);
      sg.gate_load(t0 + 2 * C, w.tok_end, lane);
    }
  }
  barrier_lds();
  if (wave == 4 && NC > 0) {
    const float x = s.lgb[0][lane];
    lsum += ws_gates(s.g[0], lane < w.tok_end - t0 ? x : 0.f, lane);
  }
  barrier_lds();

  if (state_wave) {
    // S_acc[t][r] = S[16 t + 4 lg4 + r][col0 + 16 c + ln]
    f32x4 S_acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) S_acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ci = 0; ci < NC; ++ci) {
      const int st = ci & 1;
      const WsGates &G = s.g[st];
      const uint16_t *sk = s.k[st];
      const uint16_t *sv = s.v[st];
      const float gam = G.gam;
#pragma unroll
      for (int t = 0; t < 8; ++t) S_acc[t] *= gam;
      // S += K^T (kappa . V) over keys 32 kb .. 32 kb + 31: B = kappa . V
      // (hi, lo; slot 8 lg4 + e <-> key 32 kb + 8 lg4 + e, column 16 c + ln),
      // A = K^T (the same key slots, row d = 16 t + ln)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r0 = 32 * kb + 8 * lg4 + (ln >> 2);
        const int cc = 16 * c + 4 * (ln & 3);
        const u32x2 x0 = lds_tr16(&sv[v_off(r0, cc)]);
        const u32x2 x1 = lds_tr16(&sv[v_off(r0 + 4, cc)]);
        u32x4 kt[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const u32x2 a0 = lds_tr16(&sk[qk_off<DK>(r0, 16 * t + 4 * (ln & 3))]);
          const u32x2 a1 = lds_tr16(&sk[qk_off<DK>(r0 + 4, 16 * t + 4 * (ln & 3))]);
          kt[t] = u32x4{a0.x, a0.y, a1.x, a1.y};
        }
        const u32x4 vf = u32x4{x0.x, x0.y, x1.x, x1.y};
        const f32x4 kap0 = *reinterpret_cast<const f32x4 *>(&G.kap[32 * kb + 8 * lg4]);
        const f32x4 kap1 = *reinterpret_cast<const f32x4 *>(&G.kap[32 * kb + 8 * lg4 + 4]);
        u32x4 kv_h, kv_l;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const uint32_t vw = vf[e2];
          const float v0 = __uint_as_float(vw << 16), v1 = __uint_as_float(vw & 0xffff0000u);
          const f32x4 &kk = e2 < 2 ? kap0 : kap1;
          uint32_t hh, ll;
          split_pk_bf16(kk[2 * (e2 & 1)] * v0, kk[2 * (e2 & 1) + 1] * v1, hh, ll);
          kv_h[e2] = hh;
          kv_l[e2] = ll;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) S_acc[t] = mfma16(kt[t], kv_h, S_acc[t]);
#pragma unroll
        for (int t = 0; t < 8; ++t) S_acc[t] = mfma16(kt[t], kv_l, S_acc[t]);
        // one half's operands at a time (two workgroups share a CU: 128 VGPRs)
        __builtin_amdgcn_sched_barrier(0);
      }
      // chunk ci + 1's tiles and decay arrays are ready
      barrier_lds();
    }
    float *sout = slots + ((size_t)w.state_out * H + h) * ((size_t)DK * DV);
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sout[(size_t)(16 * t + 4 * lg4 + r) * DV + col0 + 16 * c + ln] = S_acc[t][r];
    return;
  }

  // copying wavefronts
  for (int ci = 0; ci < NC; ++ci) {
    const int tc = t0 + ci * C;
    const int st = ci & 1;
    sg.commit(s, st ^ 1, iw, lane);
    if (iw == 3) sg.gate_commit(s, (ci + 2) % 3, lane);
    sg.load(tc + 2 * C, w.tok_end, iw, lane);
    if (iw == 3) sg.gate_load(tc + 3 * C, w.tok_end, lane);
    if (wave == 4 && ci + 1 < NC) {
      const float x = s.lgb[(ci + 1) % 3][lane];
      lsum += ws_gates(s.g[st ^ 1], lane < w.tok_end - tc - C ? x : 0.f, lane);
    }
    barrier_lds();
  }
  if (wave == 4 && slice == 0 && lane == 0) slot_gamma[(size_t)w.state_out * H + h] = lsum;
}

template <typename Tout, bool REV, bool DOT>
static void launch_ws_t(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                        const float *S0, float *S_T, void *o, const FwdDims &d,
                        const WorkItem *items, const int *n_items, long blocks, long pairs,
                        const float *slots, hipStream_t stream) {
  hipLaunchKernelGGL((chunk_bf16_ws_kernel<Tout, REV, DOT>), dim3(blocks), dim3(512), 0, stream,
                     q, k, v, g, S0, S_T, static_cast<Tout *>(o), items, n_items, slots, d.T,
                     d.H, d.gts, d.dv, (int)pairs, d.dot_x, d.dot_part, d.dot_stride);
}

hipError_t launch_chunk_bf16_ws(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const float *g, const float *S0, float *S_T, void *o,
                                bool out_bf16, const FwdDims &d, const WorkItem *items,
                                const int *n_items, int grid_items, const float *slots,
                                hipStream_t stream) {
  if (d.C != kW8C || d.dk != kWsDK || d.dv % kWsSW || d.hg != 1) return hipErrorInvalidValue;
  // the reversed and dot-product runs are the backward's: per-token gates, fp32 outputs
  if ((d.rev || d.dot_x) && (out_bf16 || d.gts == 0)) return hipErrorInvalidValue;
  const long pairs = (long)grid_items * d.H;
  const long blocks = pairs * (d.dv / kWsSW);
  if (blocks == 0) return hipSuccess;
  if (d.rev && d.dot_x)
    launch_ws_t<float, true, true>(q, k, v, g, S0, S_T, o, d, items, n_items, blocks, pairs,
                                   slots, stream);
  else if (d.rev)
    launch_ws_t<float, true, false>(q, k, v, g, S0, S_T, o, d, items, n_items, blocks, pairs,
                                    slots, stream);
  else if (d.dot_x)
    launch_ws_t<float, false, true>(q, k, v, g, S0, S_T, o, d, items, n_items, blocks, pairs,
                                    slots, stream);
  else if (out_bf16)
    launch_ws_t<uint16_t, false, false>(q, k, v, g, S0, S_T, o, d, items, n_items, blocks, pairs,
                                        slots, stream);
  else
    launch_ws_t<float, false, false>(q, k, v, g, S0, S_T, o, d, items, n_items, blocks, pairs,
                                     slots, stream);
  return hipGetLastError();
}

hipError_t launch_chunk_bf16_ws_state(const uint16_t *k, const uint16_t *v, const float *g,
                                      const FwdDims &d, const WorkItem *items, const int *n_items,
                                      int grid_items, float *slots, float *slot_gamma,
                                      hipStream_t stream) {
  if (d.C != kW8C || d.dk != kWsDK || d.dv % kWsSW || d.hg != 1 || !items)
    return hipErrorInvalidValue;
  const long pairs = (long)grid_items * d.H;
  const long blocks = pairs * (d.dv / kWsSW);
  if (blocks == 0) return hipSuccess;
  if (d.rev)
    hipLaunchKernelGGL((chunk_bf16_ws_state_kernel<true>), dim3(blocks), dim3(512), 0, stream, k,
                       v, g, items, n_items, slots, slot_gamma, d.T, d.H, d.gts, d.dv, (int)pairs);
  else
    hipLaunchKernelGGL((chunk_bf16_ws_state_kernel<false>), dim3(blocks), dim3(512), 0, stream, k,
                       v, g, items, n_items, slots, slot_gamma, d.T, d.H, d.gts, d.dv, (int)pairs);
  return hipGetLastError();
}

}  // namespace gla
