// One-token GLA decode step, streaming each fp32 state through HBM once.
//
// Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), "GLA mixer":
// per (sequence, head) the state decays, absorbs k^T v, and is read by q:
//     S <- exp(l) S + k^T v  (in place),   o = q S.
// The step is bandwidth-bound: 2 * d_k * d_v * 4 bytes of state move per
// (sequence, head) against 4 d_k d_v flops, so the kernel is a coalesced
// 128-bit read-modify-write stream with the d_k reduction for o done in
// registers, a cross-lane shuffle and one LDS exchange.
//
// Mapping: one 256-thread workgroup per (sequence, head). Thread t owns the
// four columns 4*(t % (dv/4)) .. +3 of the rows r0 + i*RP, r0 = t / (dv/4),
// RP = 256 / (dv/4); a wavefront therefore reads whole 512-byte (dv = 128)
// rows, and every thread issues all of its dk/RP 16-byte loads before using
// any of them, so each CU keeps many bytes in flight.
//
// Serving-pool variant (the page's "Inference optimization": one fixed-size
// state per sequence, kept in the serving engine's pool): with `slots`, the
// state of request n is S_pool[slots[n]]; a slot outside [0, P) marks a padded
// lane of a fixed-width batch, which touches no state and outputs zeros.
//
// Processing order. Workgroups start in launch order, so the requests whose
// states stream at the same time are those at neighbouring launch positions,
// and HBM3E serves the read-modify-write stream measurably faster for some
// address mixes than for others (1,280 x 16 heads of 128 x 128, one step:
// requests in order 470-480 us; in a random order of 1 MiB slots 510-517 us,
// with more DRAM credit stalls and no more address-translation misses; slots
// sorted 481 us; groups of four consecutive requests, the groups at a stride
// of three, 448-454 us; 96 x 192 heads, 1.125 MiB a request: launch order
// fastest, 538 us, groups of four 553 us). So position j serves request
// map(j): the order that gla_decode_slot_order writes, when the caller passes
// one (the pool's 4 MiB blocks of entries at the same stride, slot order
// within a block), and for a dense batch whose requests tile 4 MiB exactly,
// groups of 4 MiB at a stride coprime with their count (a permutation for
// every N); otherwise launch order.
#include <algorithm>
#include <numeric>

#include "gla_common.h"
#include "gla_internal.h"

namespace gla {

// The stride at which groups are visited: the first of 3, 5, 7, ... coprime
// with the group count (1, i.e. in place, below three groups or if none is).
static int group_stride(int ng) {
  if (ng < 3) return 1;
  for (int a : {3, 5, 7, 11, 13, 17, 19, 23})
    if (std::gcd(a, ng) == 1) return a;
  return 1;
}

// a^-1 mod m for a, m coprime and m >= 2 (extended Euclid); 0 if none exists.
static int inverse_mod(int a, int m) {
  long r0 = m, r1 = a % m, t0 = 0, t1 = 1;
  while (r1 != 0) {
    const long qt = r0 / r1, r2 = r0 - qt * r1, t2 = t0 - qt * t1;
    r0 = r1;
    r1 = r2;
    t0 = t1;
    t1 = t2;
  }
  if (r0 != 1) return 0;
  return (int)((t0 % m + m) % m);
}

// States per 4 MiB group: only where a request's (or pool entry's) states tile
// 4 MiB exactly (96 x 192 heads, 1.125 MiB a request, stream fastest in launch
// order); 0 otherwise.
static int group_size(long bytes_per_state) {
  const long group = 4l << 20;
  if (bytes_per_state <= 0 || bytes_per_state > group || group % bytes_per_state) return 0;
  return (int)(group / bytes_per_state);
}

ReqMap make_req_map(const int32_t *order, int n, long bytes_per_request) {
  ReqMap m{order, n, 1, 0, 1};
  const int gs = group_size(bytes_per_request);
  if (order || n <= 0 || gs == 0) return m;
  m.gs = gs;
  m.ng = n / m.gs;
  m.stride = group_stride(m.ng);
  return m;
}

template <int DK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void decode_step_kernel(const Tin *__restrict__ q,
                                                          const Tin *__restrict__ k,
                                                          const Tin *__restrict__ v,
                                                          const float *__restrict__ g,
                                                          float *__restrict__ S,
                                                          Tout *__restrict__ o,
                                                          const int32_t *__restrict__ slots,
                                                          int P, int H, ReqMap map) {
  constexpr int TPR = DV / 4;   // threads per state row
  constexpr int RP = 256 / TPR; // rows per pass
  constexpr int NP = DK / RP;   // passes
  static_assert(DK % RP == 0, "d_k must be a multiple of the rows per pass");
  __shared__ f32x4 red[4][TPR];

  const int pos = (int)(blockIdx.x / H);
  const int rq = map(pos);
  if (rq < 0) return;
  const size_t p = (size_t)rq * H + blockIdx.x % H;  // (sequence, head) pair
  const int t = threadIdx.x;
  const int c4 = t % TPR;
  const int r0 = t / TPR;
  size_t sp = p;  // state of this pair
  if (slots) {
    const int slot = map.slot(pos, slots, rq);
    if (slot < 0 || slot >= P) {  // padded lane
      if (t < TPR) {
        Tout *op = o + p * DV + 4 * t;
#pragma unroll
        for (int j = 0; j < 4; ++j) store_from_f32(op, j, 0.f);
      }
      return;
    }
    sp = (size_t)slot * H + p % H;
  }
  f32x4 *Sp = reinterpret_cast<f32x4 *>(S + sp * (size_t)(DK * DV));

  f32x4 s[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) s[i] = __builtin_nontemporal_load(Sp + (r0 + i * RP) * TPR + c4);

  const float gate = gate_exp(g[p]);
  f32x4 vv;
  vv.x = load_as_f32(v, p * DV + 4 * c4 + 0);
  vv.y = load_as_f32(v, p * DV + 4 * c4 + 1);
  vv.z = load_as_f32(v, p * DV + 4 * c4 + 2);
  vv.w = load_as_f32(v, p * DV + 4 * c4 + 3);
  float kk[NP], qq[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    kk[i] = load_as_f32(k, p * DK + r0 + i * RP);
    qq[i] = load_as_f32(q, p * DK + r0 + i * RP);
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    f32x4 x = gate * s[i] + kk[i] * vv;
    __builtin_nontemporal_store(x, Sp + (r0 + i * RP) * TPR + c4);
    acc += qq[i] * x;
  }

  // Sum the partial outputs of the threads that own the same columns: first
  // across the lanes of a wavefront (lanes c4, c4 + TPR, ...), then across the
  // four wavefronts through LDS.
#pragma unroll
  for (int off = TPR; off < 64; off *= 2) {
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }
  const int wave = t / 64, lane = t % 64;
  if (lane < TPR) red[wave][lane] = acc;
  __syncthreads();
  if (t < TPR) {
    f32x4 r = red[0][t] + red[1][t] + red[2][t] + red[3][t];
    Tout *op = o + p * DV + 4 * t;
    store_from_f32(op, 0, r.x);
    store_from_f32(op, 1, r.y);
    store_from_f32(op, 2, r.z);
    store_from_f32(op, 3, r.w);
  }
}

// The same step with the columns of a (sequence, head) split over
// workgroups of CW columns each (CW = d_v: one workgroup per pair). Each
// output column depends only on its own state column, so slices need no
// reduction between them: RP rows per pass of TPR = CW / 4 threads, and the
// d_k reduction of o through LDS (each thread's partial sum, then one thread
// per column group adds RP). Serves row widths whose 4-column groups do not
// divide a wavefront (d_v = 192 in Laplace 3B's 96 x 192 heads, "GLA mixer")
// and small batches, whose few (sequence, head) pairs would leave CUs idle or
// unevenly loaded.
template <int DK, int DV, int CW, int RP, typename Tin, typename Tout>
__global__ __launch_bounds__(512) void decode_step_rows_kernel(const Tin *__restrict__ q,
                                                               const Tin *__restrict__ k,
                                                               const Tin *__restrict__ v,
                                                               const float *__restrict__ g,
                                                               float *__restrict__ S,
                                                               Tout *__restrict__ o,
                                                               const int32_t *__restrict__ slots,
                                                               int P, int H, ReqMap map) {
  constexpr int TPR = CW / 4;
  constexpr int NS = DV / CW;  // column slices per pair
  constexpr int NP = DK / RP;
  static_assert(DK % RP == 0 && DV % CW == 0 && CW % 4 == 0, "row tiling");
  __shared__ f32x4 red[RP][TPR];

  const int pos = (int)(blockIdx.x / NS);  // launch position of the pair
  const int rq = map(pos / H);
  if (rq < 0) return;
  const size_t p = (size_t)rq * H + pos % H;
  const int col0 = (int)(blockIdx.x % NS) * CW;
  const int t = threadIdx.x;
  const int c4 = t % TPR;
  const int r0 = t / TPR;
  size_t sp = p;
  if (slots) {
    const int slot = map.slot(pos / H, slots, rq);
    if (slot < 0 || slot >= P) {
      if (t < TPR) {
        Tout *op = o + p * DV + col0 + 4 * t;
#pragma unroll
        for (int j = 0; j < 4; ++j) store_from_f32(op, j, 0.f);
      }
      return;
    }
    sp = (size_t)slot * H + p % H;
  }
  f32x4 *Sp = reinterpret_cast<f32x4 *>(S + sp * (size_t)(DK * DV) + col0);

  f32x4 s[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i)
    s[i] = __builtin_nontemporal_load(Sp + (r0 + i * RP) * (DV / 4) + c4);
  const float gate = gate_exp(g[p]);
  const size_t vc = p * DV + col0 + 4 * c4;
  f32x4 vv;
  vv.x = load_as_f32(v, vc + 0);
  vv.y = load_as_f32(v, vc + 1);
  vv.z = load_as_f32(v, vc + 2);
  vv.w = load_as_f32(v, vc + 3);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const float kk = load_as_f32(k, p * DK + r0 + i * RP);
    const float qq = load_as_f32(q, p * DK + r0 + i * RP);
    const f32x4 x = gate * s[i] + kk * vv;
    __builtin_nontemporal_store(x, Sp + (r0 + i * RP) * (DV / 4) + c4);
    acc += qq * x;
  }
  red[r0][c4] = acc;
  __syncthreads();
  if (t < TPR) {
    f32x4 r = red[0][t];
#pragma unroll
    for (int i = 1; i < RP; ++i) r += red[i][t];
    Tout *op = o + p * DV + col0 + 4 * t;
    store_from_f32(op, 0, r.x);
    store_from_f32(op, 1, r.y);
    store_from_f32(op, 2, r.z);
    store_from_f32(op, 3, r.w);
  }
}

// Sum over the 64 lanes of a wavefront (every lane active), returned as a
// wave-uniform value: pairs and quads by quad permutes, rows of 16 by row
// rotations, then the row broadcasts carry rows 0-1 into row 3, whose last
// lane ends with the total.
__device__ __forceinline__ float dpp_add(float x, int v) { return x + __int_as_float(v); }
__device__ __forceinline__ float wave_total(float x) {
  x = dpp_add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
  x = dpp_add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
  x = dpp_add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
  x = dpp_add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  x = dpp_add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xa, 0xf, false));
  x = dpp_add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xc, 0xf, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// One decode step followed by the token-mixer epilogue in the same workgroup
// (Laplace 3B on AWS Trainium2, "GLA mixer": the readout o of a head gets a
// gated copy of v, o' = o + sigmoid(q . (a * k)) v, then the head's RMSNorm
// and the SiLU output gate, z = o' / sqrt(mean(o'^2) + eps) * w * silu(g_out)).
// The workgroup owns the whole row of its (sequence, head), so o never leaves
// registers: the state is streamed as in decode_step_rows_kernel, the logit
// is a block sum over d_k (shuffles, then one LDS value per wavefront), and
// wavefront 0 finishes the row (its d_v / 4 <= 64 column groups) with a
// wavefront sum for the RMS.
template <int DK, int DV, int RP, typename Tin, typename Tout>
__global__ __launch_bounds__(512) void decode_mixer_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ g, float *__restrict__ S, const Tin *__restrict__ gout,
    const float *__restrict__ a, const float *__restrict__ w, float eps, Tout *__restrict__ z,
    const int32_t *__restrict__ slots, int P, int H, ReqMap map) {
  constexpr int TPR = DV / 4;
  constexpr int NP = DK / RP;
  constexpr int NW = RP * TPR / 64;  // wavefronts
  static_assert(DK % RP == 0 && DV % 4 == 0 && TPR <= 64 && (RP * TPR) % 64 == 0, "row tiling");
  __shared__ f32x4 red[RP][TPR];
  __shared__ float lred[NW];

  const int pos = (int)(blockIdx.x / H);
  const int rq = map(pos);
  if (rq < 0) return;
  const size_t p = (size_t)rq * H + blockIdx.x % H;
  const int t = threadIdx.x;
  const int c4 = t % TPR;
  const int r0 = t / TPR;
  const int h = (int)(p % H);
  size_t sp = p;
  if (slots) {
    const int slot = map.slot(pos, slots, rq);
    if (slot < 0 || slot >= P) {  // padded lane: no state touched, z = 0
      if (t < TPR) store4_from_f32(z + p * DV + 4 * t, f32x4{0.f, 0.f, 0.f, 0.f});
      return;
    }
    sp = (size_t)slot * H + h;
  }
  f32x4 *Sp = reinterpret_cast<f32x4 *>(S + sp * (size_t)(DK * DV));

  // The epilogue's own operands go out before the state stream: loads and
  // stores share one counter, so a load issued after the state stores would
  // make its first use wait for all of them.
  // Branch-free (clamped indices, unused values dropped later), so that they
  // share a basic block with the state loads and nothing waits for them early.
  const int tk = t < DK ? t : 0, tc = t < TPR ? t : 0;
  const float lq = load_as_f32(q, p * DK + tk), la = a[(size_t)h * DK + tk],
              lk = load_as_f32(k, p * DK + tk);  // the logit q . (a * k): one key channel per thread
  float go[4], wr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    go[j] = load_as_f32(gout, p * DV + 4 * tc + j);
    wr[j] = w[(size_t)h * DV + 4 * tc + j];
  }
  f32x4 s[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) s[i] = __builtin_nontemporal_load(Sp + (r0 + i * RP) * TPR + c4);
  const float gate = gate_exp(g[p]);
  const size_t vc = p * DV + 4 * c4;
  f32x4 vv;
  vv.x = load_as_f32(v, vc + 0);
  vv.y = load_as_f32(v, vc + 1);
  vv.z = load_as_f32(v, vc + 2);
  vv.w = load_as_f32(v, vc + 3);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const float kk = load_as_f32(k, p * DK + r0 + i * RP);
    const float qq = load_as_f32(q, p * DK + r0 + i * RP);
    const f32x4 x = gate * s[i] + kk * vv;
    __builtin_nontemporal_store(x, Sp + (r0 + i * RP) * TPR + c4);
    acc += qq * x;
  }
  red[r0][c4] = acc;
  // the logit, summed over the block
  const float lp = wave_total(t < DK ? lq * la * lk : 0.f);
  if (t % 64 == 0) lred[t / 64] = lp;
  __syncthreads();
  if (t < 64) {
    float logit = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) logit += lred[i];
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (t < TPR) {
#pragma unroll
      for (int i = 0; i < RP; ++i) o += red[i][t];
    }
    const float sg = 1.f / (1.f + expf(-logit));
    const f32x4 x = o + sg * vv;  // thread t < TPR owns columns 4t .. 4t+3 (c4 = t)
    const float ss = wave_total(t < TPR ? x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3] : 0.f);
    const float inv = 1.f / sqrtf(ss * (1.f / DV) + eps);
    if (t < TPR) {
      Tout *zp = z + p * DV + 4 * t;
      f32x4 zz;
#pragma unroll
      for (int j = 0; j < 4; ++j) zz[j] = x[j] * inv * wr[j] * (go[j] / (1.f + expf(-go[j])));
      store4_from_f32(zp, zz);
    }
  }
}

struct DecodeArgs {
  const void *q, *k, *v;
  const float *g;
  float *S;
  void *o;
  const int32_t *slots;
  int P, H, pairs;
  ReqMap map;
};

// pairs below this many per CU run as column slices
constexpr int kSplitPairsPerCu = 2;

template <int DK, int DV, typename Tin, typename Tout>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_step_kernel<DK, DV, Tin, Tout>), dim3(a.pairs), dim3(256), 0, stream,
                     static_cast<const Tin *>(a.q), static_cast<const Tin *>(a.k),
                     static_cast<const Tin *>(a.v), a.g, a.S, static_cast<Tout *>(a.o), a.slots,
                     a.P, a.H, a.map);
  return hipGetLastError();
}

template <int DK, int DV, int CW, int RP, typename Tin, typename Tout>
static hipError_t launch_decode_rows_t(const DecodeArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_step_rows_kernel<DK, DV, CW, RP, Tin, Tout>),
                     dim3((unsigned)a.pairs * (DV / CW)), dim3(RP * CW / 4), 0, stream,
                     static_cast<const Tin *>(a.q),
                     static_cast<const Tin *>(a.k), static_cast<const Tin *>(a.v), a.g, a.S,
                     static_cast<Tout *>(a.o), a.slots, a.P, a.H, a.map);
  return hipGetLastError();
}

template <int DK, int DV, int CW, int RP>
static hipError_t launch_decode_rows_d(const DecodeArgs &a, bool in_bf16, bool out_bf16,
                                       hipStream_t stream) {
  if (in_bf16) {
    return out_bf16 ? launch_decode_rows_t<DK, DV, CW, RP, uint16_t, uint16_t>(a, stream)
                    : launch_decode_rows_t<DK, DV, CW, RP, uint16_t, float>(a, stream);
  }
  return out_bf16 ? launch_decode_rows_t<DK, DV, CW, RP, float, uint16_t>(a, stream)
                  : launch_decode_rows_t<DK, DV, CW, RP, float, float>(a, stream);
}

template <int DK, int DV>
static hipError_t launch_decode_d(const DecodeArgs &a, bool in_bf16, bool out_bf16,
                                  hipStream_t stream) {
  if (in_bf16) {
    return out_bf16 ? launch_decode_t<DK, DV, uint16_t, uint16_t>(a, stream)
                    : launch_decode_t<DK, DV, uint16_t, float>(a, stream);
  }
  return out_bf16 ? launch_decode_t<DK, DV, float, uint16_t>(a, stream)
                  : launch_decode_t<DK, DV, float, float>(a, stream);
}

hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g, float *S,
                         void *o, int N, int H, int dk, int dv, bool in_bf16, bool out_bf16,
                         const int32_t *slots, const int32_t *order, int P, int n_cu,
                         hipStream_t stream) {
  const long pairs = (long)N * H;
  if (pairs == 0) return hipSuccess;
  const DecodeArgs a{q, k, v, g, S, o, slots, P, H, (int)pairs,
                     make_req_map(order, N, slots ? 0 : (long)H * dk * dv * 4)};
  if (pairs < (long)kSplitPairsPerCu * n_cu) {  // few pairs: 64- or 32-column slices
    if (dk == 128 && dv == 128)
      return launch_decode_rows_d<128, 128, 32, 32>(a, in_bf16, out_bf16, stream);
    if (dk == 128 && dv == 64)
      return launch_decode_rows_d<128, 64, 32, 32>(a, in_bf16, out_bf16, stream);
    if (dk == 64 && dv == 128)
      return launch_decode_rows_d<64, 128, 32, 32>(a, in_bf16, out_bf16, stream);
    if (dk == 96 && dv == 192)
      return launch_decode_rows_d<96, 192, 64, 16>(a, in_bf16, out_bf16, stream);
    return launch_decode_rows_d<64, 64, 32, 32>(a, in_bf16, out_bf16, stream);
  }
  if (dk == 128 && dv == 128) return launch_decode_d<128, 128>(a, in_bf16, out_bf16, stream);
  if (dk == 128 && dv == 64) return launch_decode_d<128, 64>(a, in_bf16, out_bf16, stream);
  if (dk == 64 && dv == 128) return launch_decode_d<64, 128>(a, in_bf16, out_bf16, stream);
  if (dk == 96 && dv == 192)
    return launch_decode_rows_d<96, 192, 192, 8>(a, in_bf16, out_bf16, stream);
  return launch_decode_d<64, 64>(a, in_bf16, out_bf16, stream);
}

template <int DK, int DV, int RP, typename Tin, typename Tout>
static hipError_t launch_mixer_t(const MixerArgs &m, hipStream_t stream) {
  hipLaunchKernelGGL((decode_mixer_kernel<DK, DV, RP, Tin, Tout>), dim3((unsigned)m.pairs),
                     dim3(RP * DV / 4), 0, stream, static_cast<const Tin *>(m.q),
                     static_cast<const Tin *>(m.k), static_cast<const Tin *>(m.v), m.g, m.S,
                     static_cast<const Tin *>(m.gout), m.a, m.w, m.eps, static_cast<Tout *>(m.z),
                     m.slots, m.P, m.H, m.map);
  return hipGetLastError();
}

template <int DK, int DV, int RP>
static hipError_t launch_mixer_d(const MixerArgs &m, bool in_bf16, bool out_bf16,
                                 hipStream_t stream) {
  if (in_bf16) {
    return out_bf16 ? launch_mixer_t<DK, DV, RP, uint16_t, uint16_t>(m, stream)
                    : launch_mixer_t<DK, DV, RP, uint16_t, float>(m, stream);
  }
  return out_bf16 ? launch_mixer_t<DK, DV, RP, float, uint16_t>(m, stream)
                  : launch_mixer_t<DK, DV, RP, float, float>(m, stream);
}

hipError_t launch_decode_mixer(const MixerArgs &m_in, int dk, int dv, bool in_bf16, bool out_bf16,
                               hipStream_t stream) {
  if (m_in.pairs == 0) return hipSuccess;
  MixerArgs m = m_in;
  m.map = make_req_map(m.slots ? m.map.order : nullptr, (int)(m.pairs / m.H),
                       m.slots ? 0 : (long)m.H * dk * dv * 4);
  if (dk == 128 && dv == 128) return launch_mixer_d<128, 128, 8>(m, in_bf16, out_bf16, stream);
  if (dk == 128 && dv == 64) return launch_mixer_d<128, 64, 16>(m, in_bf16, out_bf16, stream);
  if (dk == 64 && dv == 128) return launch_mixer_d<64, 128, 8>(m, in_bf16, out_bf16, stream);
  if (dk == 96 && dv == 192) return launch_mixer_d<96, 192, 8>(m, in_bf16, out_bf16, stream);
  if (dk == 64 && dv == 64) return launch_mixer_d<64, 64, 16>(m, in_bf16, out_bf16, stream);
  return hipErrorInvalidValue;
}

// The processing order for gla_decode_step_slots and gla_decode_mixer (order
// [2, N]: the requests, then their slots, so that a decode workgroup reads its
// slot without waiting for its request index): a counting sort of the
// requests by the key of their slot in one workgroup, with a counter per pool
// entry and one for the padded lanes (slots outside [0, P)), which go last.
// The key streams the pool the way the dense step streams a batch: the pool
// in blocks of gs entries (4 MiB of states), block b at rank b * s^-1 mod nb
// so that consecutive ranks are s blocks apart, slot order within a block,
// and the slots past the last whole block after every block, in slot order
// (gs = 0: slot order throughout). 1,280 requests on random slots of a
// 2,048-entry pool of 1 MiB states: 471 us against 478 us per step in plain
// slot order. The key is a permutation of 0 .. P-1. Requests on the same slot
// (a caller error: their updates race) are placed in any order; the result is
// a permutation of 0 .. N-1 for every input.
constexpr int kOrderThreads = 1024;

struct OrderKey {
  int gs, nb, inv;  // entries per block, whole blocks, inverse of the stride mod nb
  __device__ __forceinline__ int operator()(int sl) const {
    if (gs == 0 || sl >= gs * nb) return sl;
    const int b = sl / gs;
    return (int)(((long)b * inv) % nb) * gs + sl % gs;
  }
};

__global__ __launch_bounds__(kOrderThreads) void slot_order_kernel(const int32_t *__restrict__ slots,
                                                                   int N, int P, OrderKey key,
                                                                   int32_t *__restrict__ order) {
  extern __shared__ uint32_t cnt[];  // P + 1 counters
  __shared__ uint32_t wsum[kOrderThreads / 64];
  const int t = threadIdx.x;
  const int K = P + 1;
  for (int i = t; i < K; i += kOrderThreads) cnt[i] = 0u;
  __syncthreads();
  for (int n = t; n < N; n += kOrderThreads) {
    const int sl = slots[n];
    atomicAdd(&cnt[sl >= 0 && sl < P ? key(sl) : P], 1u);
  }
  __syncthreads();
  // exclusive prefix sum over the K counters: each thread a run of consecutive
  // counters, a block scan of the run totals, then the runs rewritten
  const int per = (K + kOrderThreads - 1) / kOrderThreads;
  const int b0 = min(K, t * per), b1 = min(K, b0 + per);
  uint32_t run = 0u;
  for (int i = b0; i < b1; ++i) run += cnt[i];
  const int lane = t % 64, wave = t / 64;
  uint32_t incl = run;
  for (int off = 1; off < 64; off *= 2) {
    const uint32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t base = 0u;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  uint32_t acc = base + incl - run;
  for (int i = b0; i < b1; ++i) {
    const uint32_t c = cnt[i];
    cnt[i] = acc;
    acc += c;
  }
  __syncthreads();
  for (int n = t; n < N; n += kOrderThreads) {
    const int sl = slots[n];
    const uint32_t pos = atomicAdd(&cnt[sl >= 0 && sl < P ? key(sl) : P], 1u);
    order[pos] = n;
    order[N + pos] = sl;
  }
}

hipError_t launch_slot_order(const int32_t *slots, int N, int P, long slot_bytes, int32_t *order,
                             hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (P < 0 || P > kMaxOrderPool) return hipErrorInvalidValue;
  OrderKey key{group_size(slot_bytes), 0, 0};
  if (key.gs > 0) {
    key.nb = P / key.gs;
    const int s = group_stride(key.nb);
    if (s > 1) key.inv = inverse_mod(s, key.nb);
    if (key.inv == 0) key = OrderKey{0, 0, 0};  // fewer than three blocks: slot order
  }
  const size_t lds = (size_t)(P + 1) * sizeof(uint32_t);
  hipLaunchKernelGGL(slot_order_kernel, dim3(1), dim3(kOrderThreads), lds, stream, slots, N, P,
                     key, order);
  return hipGetLastError();
}

}  // namespace gla
