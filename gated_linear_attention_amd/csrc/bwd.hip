// Device kernels of the chunked backward (gla_bwd_chunked).
//
// The backward of the recurrence S_t = g_t S_{t-1} + k_t^T v_t, o_t = q_t S_t
// (Laplace 3B on AWS Trainium2, automationscribe.com/?p=7116, "GLA mixer";
// training differentiates through every sequential state update, "Challenge 3:
// Backward-pass unrolling for a sequential recurrence")
// is computed from three runs of the chunked forward and the kernels below:
//  * dq_t = dO_t S_t^T is the forward output for the transposed state
//    S'_t = g_t S'_{t-1} + v_t^T k_t, i.e. the forward with (q, k, v) :=
//    (dO, v, k) and initial state S0^T;
//  * the adjoint A_u = dL/dS_u obeys A_u = g_{u+1} A_{u+1} + q_u^T dO_u from
//    A_{end-1} = q^T dO + dS_T: a forward recurrence in reversed time whose
//    gate at reversed position tau is l_{end-tau} (and 0 at tau = 0). The
//    forward kernels run it in place (their time-reversed mode reads each
//    sequence bottom-up and writes outputs back to the original rows):
//    dv_u = k_u A_u is that run with (q, k, v) := (k, q, dO) from dS_T, and
//    dk_u = v_u A_u^T the run with (q, k, v) := (v, dO, q) from dS_T^T; the
//    first of these ends in A_0, and dS0 = g_0 A_0;
//  * with B_u the cumulative log-gate, dL/dB_u = q_u.dq_u - k_u.dk_u plus
//    <dS_T, S_T> at a sequence's last token, and dl_t is the sum of dL/dB_u
//    over u >= t in the same sequence.
#include "gla_common.h"
#include "gla_internal.h"

namespace gla {

namespace {

// out[m] = in[m]^T for m = 0 .. count-1 matrices of rows x cols (fp32).
__global__ __launch_bounds__(256) void transpose_kernel(const float *__restrict__ in,
                                                        float *__restrict__ out, int rows,
                                                        int cols) {
  __shared__ float tile[32][33];
  const size_t m = blockIdx.z;
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;  // 32 x 8
  const float *a = in + m * rows * cols;
  float *b = out + m * rows * cols;
  for (int r = ty; r < 32; r += 8)
    if (r0 + r < rows && c0 + tx < cols) tile[r][tx] = a[(size_t)(r0 + r) * cols + c0 + tx];
  __syncthreads();
  for (int c = ty; c < 32; c += 8)
    if (c0 + c < cols && r0 + tx < rows) b[(size_t)(c0 + c) * rows + r0 + tx] = tile[tx][c];
}

// dB[p, h] = q.dq - k.dk for every token row (32 lanes per row, 4 elements
// per lane per step, 8 rows per workgroup). With dq2 / dk2 (the second key
// halves of split-key runs), dq += dq2 and dk += dk2 first (written back).
template <typename Tin>
__global__ __launch_bounds__(256) void gate_dot_kernel(const Tin *__restrict__ q,
                                                       const Tin *__restrict__ k,
                                                       float *__restrict__ dq,
                                                       float *__restrict__ dk,
                                                       const float *__restrict__ dq2,
                                                       const float *__restrict__ dk2,
                                                       float *__restrict__ dB, long rows, int DK) {
  const long row = (long)blockIdx.x * 8 + threadIdx.x / 32;
  const int l = threadIdx.x % 32;
  float acc = 0.f;
  if (row < rows) {
    const size_t base = (size_t)row * DK;
    for (int i = 4 * l; i < DK; i += 128) {
      const f32x4 a = load4_as_f32(q + base + i), c = load4_as_f32(k + base + i);
      f32x4 b = *reinterpret_cast<const f32x4 *>(dq + base + i);
      f32x4 d = *reinterpret_cast<const f32x4 *>(dk + base + i);
      if (dq2) {
        b += *reinterpret_cast<const f32x4 *>(dq2 + base + i);
        d += *reinterpret_cast<const f32x4 *>(dk2 + base + i);
        *reinterpret_cast<f32x4 *>(dq + base + i) = b;
        *reinterpret_cast<f32x4 *>(dk + base + i) = d;
      }
      acc += (a[0] * b[0] + a[1] * b[1]) + (a[2] * b[2] + a[3] * b[3]) -
             ((c[0] * d[0] + c[1] * d[1]) + (c[2] * d[2] + c[3] * d[3]));
    }
  }
#pragma unroll
  for (int w = 16; w > 0; w >>= 1) acc += __shfl_xor(acc, w, 32);
  if (row < rows && l == 0) dB[row] = acc;
}

// One workgroup per (sequence, head): dl = reverse cumulative sum of dB over
// the sequence (plus <dS_T, S_T> at its last token), in tiles of 2048 tokens
// from the end; and dS0 = g_0 A_0. With NP > 0 the per-token dB = q.dq -
// k.dk is formed here from the partial sums the chunk-64 forward runs wrote
// (dq_part / dk_part [NP][H][n_tok], one plane per 16-column group, read
// along the tokens); otherwise it is read from dB [token][H]. ST_t and dST_t
// are S_T^T and dS_T^T ([dv][dk]; dST_t null for dS_T = 0); A0 is the adjoint
// after the first token ([dk][dv]). dB and dl may be the same array.
//
// A reset gate at token r (g_r = 0) makes the loss independent of every
// earlier token's log-gate through tokens u >= r, and of l_r itself
// (dL/dl_r = g_r <A_r, S_{r-1}> = 0): the sum restarts at r, dl_r = 0, and
// earlier tokens sum dB over [t, r) only (the terms from r on sum to zero in
// exact arithmetic; dropping them drops their rounding). Each thread's eight
// tokens act on the running sum as run -> a run + b (a = 0 if they hold a
// reset), and the tile composes these maps from the right.
template <int NP>
__global__ __launch_bounds__(256) void gate_scan_kernel(
    const float *dB, const float *__restrict__ dq_part, const float *__restrict__ dk_part,
    long n_tok, const float *__restrict__ lg, const float *__restrict__ ST_t,
    const float *__restrict__ dST_t, const float *__restrict__ A0, float *dl,
    float *__restrict__ dS0, const int32_t *__restrict__ cu, int T, int H, int DK, int DV) {
  const int n = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x;
  // sequence bounds; packed offsets are clamped to [0, T] with e >= s (as the
  // forward's planner does), so malformed offsets stay inside the arrays
  int s, e;
  if (cu) {
    s = min(max(cu[n], 0), T);
    e = max(min(max(cu[n + 1], 0), T), s);
  } else {
    s = n * T;
    e = (n + 1) * T;
  }
  const size_t mat = (size_t)DK * DV, base = ((size_t)n * H + h) * mat;
  __shared__ float red[256], reda[256];
  __shared__ float xs[2048];
  __shared__ unsigned char fs[2048];

  // <dS_T, S_T> in 16-byte pieces (d_k d_v is a multiple of 1024), four a
  // round with all loads issued first
  const size_t n4 = mat / 4;
  float fro = 0.f;
  if (dST_t) {
    const f32x4 *a4 = reinterpret_cast<const f32x4 *>(dST_t + base);
    const f32x4 *b4 = reinterpret_cast<const f32x4 *>(ST_t + base);
    for (size_t i0 = tid; i0 < n4; i0 += 1024) {
      f32x4 a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const size_t i = i0 + 256 * u;
        a[u] = i < n4 ? a4[i] : f32x4{0.f, 0.f, 0.f, 0.f};
        b[u] = i < n4 ? b4[i] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        fro += (a[u][0] * b[u][0] + a[u][1] * b[u][1]) + (a[u][2] * b[u][2] + a[u][3] * b[u][3]);
    }
  }
  red[tid] = fro;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  fro = red[0];
  __syncthreads();

  // dS0 = g_0 A_0 (an empty sequence passes dS_T through: A_0 = dS_T)
  if (dS0) {
    float g0 = 1.f;
    if (e > s) {
      const float l0 = lg[(size_t)s * H + h];
      g0 = is_reset(l0) ? 0.f : fast_exp2(l0 * kLog2e);
    }
    const f32x4 *a4 = reinterpret_cast<const f32x4 *>(A0 + base);
    f32x4 *d4 = reinterpret_cast<f32x4 *>(dS0 + base);
    for (size_t i0 = tid; i0 < n4; i0 += 1024) {
      f32x4 a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        a[u] = i0 + 256 * u < n4 ? a4[i0 + 256 * u] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + 256 * u < n4) d4[i0 + 256 * u] = g0 * a[u];
    }
  }

  // tiles of 8 tokens per thread, last tile first; carry = the running sum
  // entering the tile from the right
  float carry = fro;
  const size_t plane = (size_t)n_tok * H;
  for (int hi = e; hi > s; hi -= 2048) {
    const int lo = hi - 2048 > s ? hi - 2048 : s;
    // the tile's dB and reset flags into LDS (the partial planes are read
    // along the tokens, every load of the tile issued before the first sum;
    // addresses clamped into the tile)
    const int cnt = hi - lo;
    float d[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const size_t t = (size_t)lo + min(tid + 256 * j, cnt - 1);
      if constexpr (NP > 0) {
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          a += dq_part[p * plane + h * (size_t)n_tok + t];
          b += dk_part[p * plane + h * (size_t)n_tok + t];
        }
        d[j] = a - b;
      } else {
        d[j] = dB[t * H + h];
      }
      l[j] = lg[t * H + h];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (tid + 256 * j < cnt) {
        xs[tid + 256 * j] = d[j];
        fs[tid + 256 * j] = is_reset(l[j]);
      }
    __syncthreads();
    // this thread's map run -> ta run + tb
    float x[8], tb = 0.f, ta = 1.f;
    bool f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = lo + 8 * tid + j < hi;
      x[j] = in ? xs[8 * tid + j] : 0.f;
      f[j] = in && fs[8 * tid + j];
    }
#pragma unroll
    for (int j = 7; j >= 0; --j) {
      if (f[j]) {
        tb = 0.f;
        ta = 0.f;
      } else {
        tb += x[j];
      }
    }
    // inclusive compositions from the right: (A, B)[tid] = map tid after maps tid+1, ...
    red[tid] = tb;
    reda[tid] = ta;
    __syncthreads();
    for (int w = 1; w < 256; w <<= 1) {
      const float yb = tid + w < 256 ? red[tid + w] : 0.f;
      const float ya = tid + w < 256 ? reda[tid + w] : 1.f;
      __syncthreads();
      red[tid] = reda[tid] * yb + red[tid];
      reda[tid] *= ya;
      __syncthreads();
    }
    // the sum entering this thread from the right, and the tile's carry out
    float run = tid < 255 ? reda[tid + 1] * carry + red[tid + 1] : carry;
    const float out = reda[0] * carry + red[0];
    __syncthreads();
#pragma unroll
    for (int j = 7; j >= 0; --j) {
      const int t = lo + 8 * tid + j;
      if (f[j]) run = 0.f;
      else run += x[j];
      if (t < hi) dl[(size_t)t * H + h] = run;
    }
    carry = out;
  }
}

}  // namespace

hipError_t launch_transpose(const float *in, float *out, int count, int rows, int cols,
                            hipStream_t stream) {
  const size_t mat = (size_t)rows * cols;
  for (int m0 = 0; m0 < count; m0 += 65535) {  // grid z is at most 65535
    const int n = count - m0 < 65535 ? count - m0 : 65535;
    hipLaunchKernelGGL(transpose_kernel, dim3((cols + 31) / 32, (rows + 31) / 32, n), dim3(256),
                       0, stream, in + m0 * mat, out + m0 * mat, rows, cols);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_dgate(const void *q, const void *k, float *dq, float *dk, const float *lg,
                        const float *ST_t, const float *dST_t, const float *A0, float *dl,
                        float *dS0, const int32_t *cu, int N, int T, int H, int DK, int DV,
                        bool in_bf16, const float *dq_part, const float *dk_part, int n_part,
                        hipStream_t stream, const float *dq2, const float *dk2) {
  if ((dq2 == nullptr) != (dk2 == nullptr) || (dq2 && n_part != 0)) return hipErrorInvalidValue;
  if (((long)DK * DV) % 1024) return hipErrorInvalidValue;  // the scan's 16-byte state pieces
  const long rows = (long)(cu ? T : (long)N * T) * H;  // token rows of the batch
  if (rows > 0 && n_part == 0) {
    const dim3 grid((unsigned)((rows + 7) / 8)), block(256);
    if (in_bf16)
      hipLaunchKernelGGL(gate_dot_kernel<uint16_t>, grid, block, 0, stream,
                         static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k), dq,
                         dk, dq2, dk2, dl, rows, DK);
    else
      hipLaunchKernelGGL(gate_dot_kernel<float>, grid, block, 0, stream,
                         static_cast<const float *>(q), static_cast<const float *>(k), dq, dk, dq2,
                         dk2, dl, rows, DK);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((long)N * H == 0) return hipSuccess;
  auto kern = n_part == 8 ? gate_scan_kernel<8> : n_part == 4 ? gate_scan_kernel<4>
                                                                : gate_scan_kernel<0>;
  if (n_part != 0 && n_part != 4 && n_part != 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)(N * H)), dim3(256), 0, stream, dl, dq_part, dk_part,
                     cu ? (long)T : (long)N * T, lg, ST_t, dST_t, A0, dl, dS0, cu, T, H, DK, DV);
  return hipGetLastError();
}

}  // namespace gla
