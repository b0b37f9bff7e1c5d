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
// Rows of 64 or 128 channels pack 4 or 2 rows per wavefront; a 192-channel
// row takes 48 lanes of one wavefront (the other 16 add zeros). Each lane
// group handles two rows, RPW apart (a wavefront covers 2 RPW consecutive rows).
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

template <int DK, int DV, typename To, typename Tin, typename Tout>
hipError_t launch_epi_t(const void *o, const void *q, const void *k, const void *v,
                        const void *g, const float *a, const float *w, float eps, void *z,
                        long n_rows, int H, hipStream_t stream) {
  constexpr int LPR = DV / 4;
  constexpr int RPW = LPR <= 32 ? 64 / LPR : 1;
  const long per_block = 4L * RPW * kEpiUnroll;
  const long blocks = (n_rows + per_block - 1) / per_block;
  hipLaunchKernelGGL((mixer_epilogue_kernel<DK, DV, To, Tin, Tout>), dim3((unsigned)blocks),
                     dim3(256), 0, stream, static_cast<const To *>(o),
                     static_cast<const Tin *>(q), static_cast<const Tin *>(k),
                     static_cast<const Tin *>(v), static_cast<const Tin *>(g), a, w, eps,
                     static_cast<Tout *>(z), n_rows, H);
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
