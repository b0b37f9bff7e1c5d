// Token-mixer epilogue around the GLA readout, one pass over HBM.
//
// Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), "GLA mixer":
// after the state readout o of a head, a gated copy of the value is added
// (self-augmentation; the gate is the sigmoid of q dotted with a learned
// per-channel rescaling a of k), each head's outputs pass through an RMSNorm
// whose weights its decay tier shares, and the result is gated by SiLU of
// the gate stream g:
//     o' = o + sigmoid(sum_i q_i a_i k_i) v
//     z  = o' / sqrt(mean(o'^2) + eps) * w_h * silu(g)
// Per (token, head) row this reads o, q, k, v, g and writes z once; a and w
// (per head) stay in cache. Bandwidth-bound: a row is d_v / 4 lanes, each
// with four consecutive channels (16-byte fp32 or 8-byte bf16 accesses) and
// d_k / (d_v / 4) key channels; the two row reductions (the logit and the
// sum of squares) are cross-lane shuffles inside the row's lane group.
// Rows of 64 or 128 channels pack 4 or 2 rows per wavefront. Each lane group
// handles two rows, RPW apart (a wavefront covers 2 RPW consecutive rows).
// 192-channel rows use a layout of their own (mixer_epilogue_r16_kernel).
#include "gla_common.h"
#include "gla_internal.h"

namespace gla {

namespace {

// Streaming accesses (each byte is read or written once): non-temporal.
__device__ __forceinline__ f32x4 ld4(const float *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
__device__ __forceinline__ f32x4 ld4(const uint16_t *p) {
  const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
               __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
}
__device__ __forceinline__ void st4(float *p, const f32x4 &x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
}
__device__ __forceinline__ void st4(uint16_t *p, const f32x4 &x) {
  u32x2 w;
  w.x = cvt_pk_bf16(x[0], x[1]);
  w.y = cvt_pk_bf16(x[2], x[3]);
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(p));
}

template <int N, typename T>
__device__ __forceinline__ void ldn(const T *p, float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    const f32x4 t = load4_as_f32(p + i);
    x[i] = t[0];
    x[i + 1] = t[1];
    x[i + 2] = t[2];
    x[i + 3] = t[3];
  }
}
template <> __device__ __forceinline__ void ldn<2, float>(const float *p, float (&x)[2]) {
  const f32x2 t = *reinterpret_cast<const f32x2 *>(p);
  x[0] = t[0];
  x[1] = t[1];
}
template <> __device__ __forceinline__ void ldn<2, uint16_t>(const uint16_t *p, float (&x)[2]) {
  const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
  x[0] = __uint_as_float(w << 16);
  x[1] = __uint_as_float(w & 0xffff0000u);
}

// Sum over the G lanes of a lane group (G a power of two dividing 64, or 64).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

// Rows per lane group, all of their loads issued before the first is used
// (two measured 10% faster than one, with the non-temporal accesses, on the
// 96 x 192 shape; four were slower).
constexpr int kEpiUnroll = 2;

template <int DK, int DV, typename To, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void mixer_epilogue_kernel(
    const To *o, const Tin *__restrict__ q, const Tin *__restrict__ k,
    const Tin *__restrict__ v, const Tin *__restrict__ g, const float *__restrict__ a,
    const float *__restrict__ w, float eps, Tout *z, long n_rows, int H) {
  // z may be o itself (same dtype): every lane reads its o elements before it
  // writes the same elements of z.
  constexpr int LPR = DV / 4;                  // lanes per row
  constexpr int RPW = LPR <= 32 ? 64 / LPR : 1;  // rows per wavefront
  constexpr int GL = LPR <= 32 ? LPR : 64;     // lanes of one reduction group
  constexpr int EK = DK / LPR;                 // key channels per lane
  constexpr int U = kEpiUnroll;
  static_assert(DV % 4 == 0 && DK % LPR == 0 && (EK == 2 || EK % 4 == 0), "row layout");
  const int lane = threadIdx.x % 64;
  const int li = lane % GL;  // lane within the row group
  const long row0 = ((long)blockIdx.x * 4 + threadIdx.x / 64) * RPW * U + lane / GL;

  float dot[U];
  f32x4 ov[U], vv[U], gv[U], wv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const long row = row0 + (long)u * RPW;
    const bool active = li < LPR && row < n_rows;
    const int h = (int)(row % H);
    dot[u] = 0.f;
    ov[u] = vv[u] = gv[u] = wv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (active) {
      const size_t rv = (size_t)row * DV + 4 * li, rk = (size_t)row * DK + EK * li;
      float qe[EK], ke[EK], ae[EK];
      ldn<EK>(q + rk, qe);
      ldn<EK>(k + rk, ke);
      ldn<EK>(a + (size_t)h * DK + EK * li, ae);
      ov[u] = ld4(o + rv);
      vv[u] = ld4(v + rv);
      gv[u] = ld4(g + rv);
      wv[u] = load4_as_f32(w + (size_t)h * DV + 4 * li);
#pragma unroll
      for (int e = 0; e < EK; ++e) dot[u] += qe[e] * ae[e] * ke[e];
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const long row = row0 + (long)u * RPW;
    const float s = sigmoid_f(group_sum<GL>(dot[u]));
    const f32x4 x = ov[u] + s * vv[u];
    float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
    ss = group_sum<GL>(ss);
    const float inv = 1.f / sqrtf(ss * (1.f / DV) + eps);
    if (li < LPR && row < n_rows) {
      f32x4 r;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = x[j] * inv * wv[u][j] * (gv[u][j] * sigmoid_f(gv[u][j]));
      st4(z + (size_t)row * DV + 4 * li, r);
    }
  }
}

// Sum over the 16 lanes of a DPP row (pairs and quads by quad permutes, then
// row rotations by 4 and 8); every lane of the row ends with the sum. All 64
// lanes must be active.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  return x;
}

// Two consecutive key channels (4-byte bf16 pair or 8-byte fp32 pair).
__device__ __forceinline__ f32x2 ld2(const float *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x2 *>(p));
}
__device__ __forceinline__ f32x2 ld2(const uint16_t *p) {
  const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
  return f32x2{__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
}

// Rows per 16-lane group in the kernel below: one (with their loads, a lane
// already has 12 value and 6 key channels in flight; two, three and four rows
// measured 3%, 6% and 8% slower).
constexpr int kR16Rows = 1;

// 192-channel rows (the Laplace heads), where d_v / 4 = 48 lanes per row would
// leave 16 of 64 idle: a (token, head) row is one DPP row of 16 lanes, four
// rows per wavefront (11% faster on laplace_2k; slower for 64- and
// 128-channel rows, whose lane groups are already full). Lane l of a row
// holds value channels 64 j + 4 l .. +3 (j < d_v / 64: each piece index j is
// one contiguous 256-byte fp32 / 128-byte bf16 span of the row across the 16
// lanes) and key channels 32 j + 2 l, +1 (j < d_k / 32); the two row sums
// are four DPP steps each.
template <int DK, int DV, typename To, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void mixer_epilogue_r16_kernel(
    const To *o, const Tin *__restrict__ q, const Tin *__restrict__ k,
    const Tin *__restrict__ v, const Tin *__restrict__ g, const float *__restrict__ a,
    const float *__restrict__ w, float eps, Tout *z, long n_rows, int H) {
  // z may be o itself (same dtype): every lane reads its o elements before it
  // writes the same elements of z.
  constexpr int CV = DV / 64;  // 4-channel value pieces per lane
  constexpr int CK = DK / 32;  // 2-channel key pieces per lane
  constexpr int U = kR16Rows;
  static_assert(DV % 64 == 0 && DK % 32 == 0, "row layout");
  const int lane = threadIdx.x % 64;
  const int li = lane % 16;
  const long row0 = ((long)blockIdx.x * 4 + threadIdx.x / 64) * 4 * U + lane / 16;

  float dot[U];
  f32x4 ov[U][CV], vv[U][CV], gv[U][CV], wv[U][CV];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const long row = row0 + 4L * u;
    dot[u] = 0.f;
#pragma unroll
    for (int j = 0; j < CV; ++j) ov[u][j] = vv[u][j] = gv[u][j] = wv[u][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (row < n_rows) {
      const int h = (int)(row % H);
#pragma unroll
      for (int j = 0; j < CK; ++j) {
        const size_t c = 32 * j + 2 * li;
        const f32x2 qe = ld2(q + (size_t)row * DK + c), ke = ld2(k + (size_t)row * DK + c);
        const f32x2 ae = *reinterpret_cast<const f32x2 *>(a + (size_t)h * DK + c);
        dot[u] += qe[0] * ae[0] * ke[0];
        dot[u] += qe[1] * ae[1] * ke[1];
      }
#pragma unroll
      for (int j = 0; j < CV; ++j) {
        const size_t c = 64 * j + 4 * li;
        ov[u][j] = ld4(o + (size_t)row * DV + c);
        vv[u][j] = ld4(v + (size_t)row * DV + c);
        gv[u][j] = ld4(g + (size_t)row * DV + c);
        wv[u][j] = load4_as_f32(w + (size_t)h * DV + c);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const long row = row0 + 4L * u;
    const float s = sigmoid_f(row16_sum(dot[u]));
    f32x4 x[CV];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < CV; ++j) {
      x[j] = ov[u][j] + s * vv[u][j];
      ss += x[j][0] * x[j][0] + x[j][1] * x[j][1] + x[j][2] * x[j][2] + x[j][3] * x[j][3];
    }
    ss = row16_sum(ss);
    const float inv = 1.f / sqrtf(ss * (1.f / DV) + eps);
    if (row < n_rows) {
#pragma unroll
      for (int j = 0; j < CV; ++j) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r[e] = x[j][e] * inv * wv[u][j][e] * (gv[u][j][e] * sigmoid_f(gv[u][j][e]));
        st4(z + (size_t)row * DV + 64 * j + 4 * li, r);
      }
    }
  }
}

template <int DK, int DV, typename To, typename Tin, typename Tout>
hipError_t launch_epi_t(const void *o, const void *q, const void *k, const void *v,
                        const void *g, const float *a, const float *w, float eps, void *z,
                        long n_rows, int H, hipStream_t stream) {
  if constexpr (DV == 192) {
    const long per_block = 16L * kR16Rows;  // four wavefronts of four row groups
    const long blocks = (n_rows + per_block - 1) / per_block;
    hipLaunchKernelGGL((mixer_epilogue_r16_kernel<DK, DV, To, Tin, Tout>),
                       dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<const To *>(o),
                       static_cast<const Tin *>(q), static_cast<const Tin *>(k),
                       static_cast<const Tin *>(v), static_cast<const Tin *>(g), a, w, eps,
                       static_cast<Tout *>(z), n_rows, H);
  } else {
    constexpr int LPR = DV / 4;
    constexpr int RPW = LPR <= 32 ? 64 / LPR : 1;
    const long per_block = 4L * RPW * kEpiUnroll;
    const long blocks = (n_rows + per_block - 1) / per_block;
    hipLaunchKernelGGL((mixer_epilogue_kernel<DK, DV, To, Tin, Tout>), dim3((unsigned)blocks),
                       dim3(256), 0, stream, static_cast<const To *>(o),
                       static_cast<const Tin *>(q), static_cast<const Tin *>(k),
                       static_cast<const Tin *>(v), static_cast<const Tin *>(g), a, w, eps,
                       static_cast<Tout *>(z), n_rows, H);
  }
  return hipGetLastError();
}

template <int DK, int DV, typename To, typename Tin>
hipError_t launch_epi_out(bool out_bf16, const void *o, const void *q, const void *k,
                          const void *v, const void *g, const float *a, const float *w, float eps,
                          void *z, long n_rows, int H, hipStream_t stream) {
  if (out_bf16)
    return launch_epi_t<DK, DV, To, Tin, uint16_t>(o, q, k, v, g, a, w, eps, z, n_rows, H, stream);
  return launch_epi_t<DK, DV, To, Tin, float>(o, q, k, v, g, a, w, eps, z, n_rows, H, stream);
}

template <int DK, int DV>
hipError_t launch_epi_d(bool o_bf16, bool in_bf16, bool out_bf16, const void *o, const void *q,
                        const void *k, const void *v, const void *g, const float *a,
                        const float *w, float eps, void *z, long n_rows, int H,
                        hipStream_t stream) {
  if (o_bf16) {
    if (in_bf16)
      return launch_epi_out<DK, DV, uint16_t, uint16_t>(out_bf16, o, q, k, v, g, a, w, eps, z,
                                                         n_rows, H, stream);
    return launch_epi_out<DK, DV, uint16_t, float>(out_bf16, o, q, k, v, g, a, w, eps, z, n_rows,
                                                    H, stream);
  }
  if (in_bf16)
    return launch_epi_out<DK, DV, float, uint16_t>(out_bf16, o, q, k, v, g, a, w, eps, z, n_rows,
                                                    H, stream);
  return launch_epi_out<DK, DV, float, float>(out_bf16, o, q, k, v, g, a, w, eps, z, n_rows, H,
                                               stream);
}

}  // namespace

hipError_t launch_mixer_epilogue(const void *o, const void *q, const void *k, const void *v,
                                 const void *g, const float *a, const float *w, float eps,
                                 void *z, long n_rows, int H, int dk, int dv, bool o_bf16,
                                 bool in_bf16, bool out_bf16, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
#define GLA_EPI(DK_, DV_)                                                                      \
  if (dk == DK_ && dv == DV_)                                                                  \
    return launch_epi_d<DK_, DV_>(o_bf16, in_bf16, out_bf16, o, q, k, v, g, a, w, eps, z,      \
                                  n_rows, H, stream);
  GLA_EPI(64, 64)
  GLA_EPI(64, 128)
  GLA_EPI(128, 64)
  GLA_EPI(128, 128)
  GLA_EPI(96, 192)
#undef GLA_EPI
  return hipErrorInvalidValue;
}

}  // namespace gla
