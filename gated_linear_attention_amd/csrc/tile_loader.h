// HBM -> LDS tile loader shared by the bf16 chunked-forward kernels (gfx950):
// 64-token chunks of Q, K (d_k wide) and a V column slice, swizzled in LDS,
// and the log-gates two chunks ahead.
#pragma once

#include "bf16_blocks.h"

namespace gla {

namespace {

constexpr int kW8C = 64;  // chunk size of the bf16 kernels

// HBM -> LDS copy of one chunk into stage st, done by NCG loading wavefronts
// (the callers pass their index among those, 0 .. NCG-1; the others return).
// Tiles are swizzled (qk_off, v_off_sw in bf16_blocks.h) so that operand reads
// of 16 consecutive rows hit distinct LDS banks. The row pointers
// advance by one chunk per next() call, so a chunk costs a few scalar adds and
// one clamp of the descriptor ranges. The log-gates go to a three-slot ring
// two chunks ahead of their use.
//
// REV (time-reversed run, used by the backward): logical token t of a
// sequence [sb, se) is memory row sb + se - 1 - t, so a chunk's rows are read
// bottom-up into the same LDS layout, and the gate at logical position
// u = t - sb is the log-gate of memory row se - u (u >= 1; 0 at u = 0). Rows
// past a chunk's end get an offset beyond the descriptor range (zeros).
template <int DK, int NCG, bool SP, bool REV = false>
struct W8Loader {
  static constexpr int C = kW8C;
  static constexpr int LW = NCG;  // loading wavefronts
  static constexpr int SW = 16 * NCG;
  static constexpr int CPR = DK / 8;
  static constexpr int QB = C * DK * 2 / 1024;  // 1 KB blocks per Q/K tile (8, 12 or 16)
  static constexpr int RPB = 1024 / (DK * 2);
  static constexpr int VB = C * SW * 2 / 1024;  // 8 or 12
  static_assert(QB % LW == 0 && VB % LW == 0, "blocks per loading wavefront");
  const uint16_t *qp, *kp, *vp;  // first row (this head / slice) of the next chunk to load
  const float *gp;               // first gate of the next gate chunk to load
  size_t qk_step, v_step, g_step;  // elements per chunk
  i32x4 rq, rk, rv, rg;
  uint32_t qk_row, v_row, g_row;   // bytes per token
  int st;
  bool active, g_active;
  // REV: head / slice bases, sb + se, the sequence start, and the current chunk's row count
  const uint16_t *qh, *kh, *vh;
  const float *gh;
  int se_sum, seq_b, n_ld, n_g;
  static constexpr int kFar = 0x7fff0000;  // an offset past any descriptor range

  // q and k have H heads (h is this workgroup's); v and the gates have HR =
  // H / (head group) heads, of which this workgroup's is hr (see the kernel).
  __device__ __forceinline__ void init(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                       const float *lg, int t0, int H, int HR, int gts, int h,
                                       int hr, int DV, int col0, int sb = 0, int se = 0) {
    if constexpr (REV) {
      qh = q + (size_t)h * DK;
      kh = k + (size_t)h * DK;
      vh = v + (size_t)hr * DV + col0;
      gh = lg + hr;
      se_sum = sb + se;
      seq_b = sb;
    }
    const size_t tok0 = (size_t)t0 * H + h;
    qp = q + tok0 * DK;
    kp = k + tok0 * DK;
    vp = v + ((size_t)t0 * HR + hr) * DV + col0;
    gp = lg + (size_t)t0 * gts + hr;
    qk_step = (size_t)C * H * DK;
    v_step = (size_t)C * HR * DV;
    g_step = (size_t)C * gts;
    qk_row = (uint32_t)H * DK * 2;
    v_row = (uint32_t)HR * DV * 2;
    g_row = (uint32_t)gts * 4;
  }
  // Descriptors for the tile chunk that starts at token t0 (the one after the
  // previous call's), to be written into stage `stage`.
  __device__ __forceinline__ void next(int t0, int tok_end, int stage) {
    active = t0 < tok_end;
    st = stage;
    if (!active) return;
    const uint32_t last = (uint32_t)(min(C, tok_end - t0) - 1);
    if constexpr (REV) {  // lowest memory row of the chunk: sb + se - t0 - n
      n_ld = (int)last + 1;
      const size_t lo = (size_t)(se_sum - t0 - n_ld);
      qp = qh + lo * (qk_row / 2);
      kp = kh + lo * (qk_row / 2);
      vp = vh + lo * (v_row / 2);
    }
    rk = make_rsrc(kp, last * qk_row + DK * 2);
    if (!SP) rq = make_rsrc(qp, last * qk_row + DK * 2);
    rv = make_rsrc(vp, last * v_row + SW * 2);
    qp += qk_step;
    kp += qk_step;
    vp += v_step;
  }
  // The same for the gate chunk starting at t0 (with a per-token gate stream,
  // gates past the end read as 0; a fixed decay reads one value for all lanes
  // and the scan masks the lanes past the end).
  __device__ __forceinline__ void gate_next(int t0, int tok_end) {
    g_active = t0 < tok_end;
    if (!g_active) return;
    const uint32_t last = (uint32_t)(min(C, tok_end - t0) - 1);
    if constexpr (REV) {  // rows se - u for u = t0 - sb + n - 1 .. t0 - sb; u = 0 is out of range
      n_g = (int)last + 1;
      rg = make_rsrc(gh + (size_t)(se_sum - t0 - n_g + 1) * (g_row / 4),
                     last * g_row + (t0 == seq_b ? 0 : 4));
      return;
    }
    rg = make_rsrc(gp, last * g_row + 4);
    gp += g_step;
  }
  template <typename Tiles>
  __device__ __forceinline__ void qk_part(Tiles &dst, i32x4 r, int wave, int lane) {
    if (wave >= LW) return;
#pragma unroll
    for (int i = 0; i < QB / LW; ++i) {
      const int blk = wave * (QB / LW) + i;
      int row, c;
      if constexpr (DK == 96) {  // rows straddle the 1 KB blocks: map the linear chunk index
        const int e = blk * 64 + lane;
        row = e / CPR;
        c = (e % CPR) ^ qk_swz<DK>(row);
      } else {
        row = blk * RPB + lane / CPR;
        c = (lane % CPR) ^ (row & (CPR - 1));
      }
      int vo = row * qk_row + c * 16;
      if constexpr (REV) vo = row < n_ld ? (n_ld - 1 - row) * qk_row + c * 16 : kFar;
      buffer_load_to_lds(r, (lds_u32 *)&dst[st][blk * 512], 16, vo, 0, 0, 0);
    }
  }
  template <class LDS>
  __device__ __forceinline__ void k_part(LDS &s, int wave, int lane) {
    if (active) qk_part(s.k, rk, wave, lane);
  }
  template <class LDS>
  __device__ __forceinline__ void q_part(LDS &s, int wave, int lane) {
    if (!SP && active) qk_part(s.q, rq, wave, lane);
  }
  template <class LDS>
  __device__ __forceinline__ void v_part(LDS &s, int wave, int lane) {
    if (!active || wave >= LW) return;
#pragma unroll
    for (int i = 0; i < VB / LW; ++i) {
      const int blk = wave * (VB / LW) + i;
      int r, c;
      if constexpr (SW == 64) {
        r = blk * 8 + lane / 8;
        c = (lane % 8) ^ (r & 7);
      } else {
        const int e = blk * 64 + lane;
        r = e / 12;
        c = (e % 12) ^ qk_swz<96>(r);
      }
      int vo = r * v_row + c * 16;
      if constexpr (REV) vo = r < n_ld ? (n_ld - 1 - r) * v_row + c * 16 : kFar;
      buffer_load_to_lds(rv, (lds_u32 *)&s.v[st][blk * 512], 16, vo, 0, 0, 0);
    }
  }
  template <class LDS>
  __device__ __forceinline__ void g_part(LDS &s, int wave, int lane, int slot) {
    if (g_active && wave == LW - 1) {
      int vo = lane * g_row;
      if constexpr (REV) vo = lane < n_g ? (n_g - 1 - lane) * g_row : kFar;
      buffer_load_to_lds(rg, (lds_u32 *)&s.lgb[slot][0], 4, vo, 0, 0, 0);
    }
  }
};

}  // namespace

}  // namespace gla
