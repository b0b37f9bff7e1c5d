// Building blocks shared by the bf16 chunked-forward kernels (gfx950).
#pragma once

#include "gla_common.h"
#include "gla_internal.h"

namespace gla {


constexpr int kBfSlice = 64;  // state columns per workgroup slice (four column groups of 16)

typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LLVM's raw buffer load that writes LDS (M0 + lane * size) instead of VGPRs.
__device__ void buffer_load_to_lds(i32x4 rsrc, lds_u32 *lds, int size, int voffset, int soffset,
                                   int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Raw buffer descriptor: 48-bit base, stride 0, range num_bytes (loads at or
// beyond it return 0), gfx9 data format word.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)((a >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane((int32_t)num_bytes);
  r.w = 0x00020000;
  return r;
}

// Workgroup barrier that orders LDS only (outstanding global loads stay in flight).
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Barrier after this wavefront's global loads (including those into LDS) landed.
__device__ __forceinline__ void barrier_all() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// The same, except that up to two vector-memory operations may still be in
// flight: for the caller to use only where those are stores issued after all
// of this wavefront's loads had completed (loads and stores share the counter
// and may complete out of order).
__device__ __forceinline__ void barrier_all_but_2() {
  asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// 16 x 16 x 16 step: lane (m, g) holds k-slots 4g .. 4g+3 of A row m and of B column m.
__device__ __forceinline__ f32x4 mfma16k16(const u32x2 &a, const u32x2 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ WorkItem bf_item_for(const WorkItem *items, int it, int T) {
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

// Element offsets in the swizzled tiles: 16-byte chunk c of row r sits at chunk
// c ^ qk_swz(r). With a power-of-two count of chunks per row the mask is
// r mod chunks-per-row. A 96-wide row (12 chunks, a 48-dword pitch, so rows r
// and r + 2 start on the same bank) keeps each chunk inside its group of four
// and uses the mask (r / 2) mod 4: the 16-byte reads of 8 consecutive rows at
// one logical chunk then cover all 32 banks.
template <int DK>
__device__ __forceinline__ int qk_swz(int r) {
  constexpr int CPR = DK / 8;
  static_assert(DK == 96 || (CPR & (CPR - 1)) == 0, "row width");
  if constexpr (DK == 96) return (r >> 1) & 3;
  else return r & (CPR - 1);
}
template <int DK>
__device__ __forceinline__ int qk_off(int r, int col) {
  if constexpr (DK == 96) return r * DK + (((col >> 3) ^ qk_swz<DK>(r)) << 3) + (col & 7);
  else return r * DK + ((((col >> 3) ^ r) & (DK / 8 - 1)) << 3) + (col & 7);
}
__device__ __forceinline__ int v_off(int r, int col) {
  return r * kBfSlice + ((((col >> 3) ^ r) & 7) << 3) + (col & 7);
}
// V tiles of SW columns: 64 as above; 96 (twelve chunks per row) swizzled like
// the 96-wide Q/K rows.
template <int SW>
__device__ __forceinline__ int v_off_sw(int r, int col) {
  static_assert(SW == 64 || SW == 96, "slice width");
  if constexpr (SW == 64) return v_off(r, col);
  else return r * SW + (((col >> 3) ^ qk_swz<96>(r)) << 3) + (col & 7);
}

__device__ __forceinline__ u32x2 lds_tr16(const uint16_t *p) {
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
  return __builtin_bit_cast(u32x2, x);
}

// The same transpose read issued as inline assembly. The compiler's wait
// insertion treats the builtin above as a read that may overlap any LDS
// direct load still in flight and waits for all outstanding global loads
// before it; these reads never touch a tile that is being loaded. The result
// is not ready until an lgkmcnt wait: pass it through lds_wait() (or
// lds_after_wait() behind a barrier that waited) before use.
__device__ __forceinline__ u32x2 lds_tr16_nowait(const uint16_t *p) {
  const uint32_t a = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint16_t *)p);
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(a));
  return r;
}
// Plain LDS reads and a store issued as inline assembly, for code that has LDS
// direct loads in flight to other buffers (see lds_tr16_nowait); a read's
// result must pass through lds_wait() before use.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char *)p);
}
__device__ __forceinline__ u32x4 lds_ld128(const void *p) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
  return r;
}
__device__ __forceinline__ uint32_t lds_ld32(const void *p) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
  return r;
}
__device__ __forceinline__ void lds_st128(void *p, const f32x4 &v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_st32(void *p, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
// Wait until at most n (0, 1, 10 or 11; anything else waits for all) of this
// wavefront's vector-memory operations are outstanding.
__device__ __forceinline__ void wait_vm_at_most(int n) {
  if (n == 11) asm volatile("s_waitcnt vmcnt(11)" ::: "memory");
  else if (n == 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// Wait for this wavefront's LDS reads; the operands are tied so that their
// users cannot be scheduled above the wait.
__device__ __forceinline__ void lds_wait(u32x4 &a) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a));
}
__device__ __forceinline__ void lds_wait(uint32_t &a) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a));
}
__device__ __forceinline__ void lds_wait(uint32_t &a, uint32_t &b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void lds_wait(uint32_t &a, uint32_t &b, uint32_t &c) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c));
}
__device__ __forceinline__ void lds_wait(u32x4 &a, u32x4 &b, u32x4 &c, u32x4 &d) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void lds_wait(u32x4 &a, u32x4 &b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void lds_wait(u32x4 &a, u32x4 &b, u32x4 &c) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c));
}
// Order values behind an lgkmcnt wait that already happened (e.g. in a barrier).
__device__ __forceinline__ void lds_after_wait(u32x4 &a, u32x4 &b, u32x4 &c, u32x4 &d) {
  asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void lds_after_wait(u32x4 &a, u32x4 &b, u32x4 &c) {
  asm volatile("" : "+v"(a), "+v"(b), "+v"(c));
}
// Tell the compiler's wait insertion that every counter is drained (emits a
// wait that is a no-op at run time when placed after barrier_all()).
__device__ __forceinline__ void counters_drained() { __builtin_amdgcn_s_waitcnt(0); }
// gfx9 s_waitcnt immediate: vmcnt(2) expcnt(7) lgkmcnt(0).
__device__ __forceinline__ void counters_drained_but_2() { __builtin_amdgcn_s_waitcnt(0x0072); }
// The same with four stores allowed in flight (vmcnt(4)).
__device__ __forceinline__ void barrier_all_but_4() {
  asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void counters_drained_but_4() { __builtin_amdgcn_s_waitcnt(0x0074); }

// Inclusive prefix sum across the 64 lanes of a wavefront with DPP row shifts
// and row broadcasts (no LDS round trips).
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  int v = __float_as_int(x);
  v = __float_as_int(__int_as_float(v) +
                     __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true)));
  v = __float_as_int(__int_as_float(v) +
                     __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true)));
  v = __float_as_int(__int_as_float(v) +
                     __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true)));
  v = __float_as_int(__int_as_float(v) +
                     __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true)));
  v = __float_as_int(__int_as_float(v) +
                     __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false)));
  v = __float_as_int(__int_as_float(v) +
                     __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false)));
  return __int_as_float(v);
}

// Last set bit of `mask` at or below bit `lane` (-1 if none): with bit p set
// where gate position p of a wavefront is a reset, the last reset at or
// before position `lane`.
__device__ __forceinline__ int last_set_upto(uint64_t mask, int lane) {
  const uint64_t upto = mask & ((2ull << lane) - 1ull);  // lane 63: every bit
  return upto ? 63 - __builtin_clzll(upto) : -1;
}
__device__ __forceinline__ int last_set(uint64_t mask) {
  return mask ? 63 - __builtin_clzll(mask) : -1;
}

// Score tile index -> (row tile ti, column tile tj), tj <= ti, row-major over
// the lower triangle (t = ti (ti + 1) / 2 + tj). Branch-free so that it folds
// to constants once the tile loop is unrolled.
__host__ __device__ constexpr int tile_ti(int t) {
  return (t >= 1) + (t >= 3) + (t >= 6) + (t >= 10) + (t >= 15) + (t >= 21) + (t >= 28);
}
__host__ __device__ constexpr int tile_tj(int t) { return t - tile_ti(t) * (tile_ti(t) + 1) / 2; }
static_assert(tile_ti(9) == 3 && tile_tj(9) == 3 && tile_ti(35) == 7 && tile_tj(30) == 2,
              "lower-triangle tile numbering");

}  // namespace gla
