// C ABI of libgla.so: argument validation, work planning and kernel launches.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <initializer_list>

#include "gla.h"
#include "gla_internal.h"

using namespace gla;

namespace {

constexpr int kMaxDevices = 64;
// cache of each device's CU count (a device constant): threads that race on
// an entry all store the same value, through atomics
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

size_t dtype_size(gla_dtype t) { return t == GLA_BF16 ? 2 : 4; }

// Tensors that the kernels read or write in 8- or 16-byte pieces, or copy
// straight into LDS, must start on a 16-byte boundary; the per-token scalar
// streams (log-gates, their gradient, sequence offsets, slots) on their
// element size. NULL passes both.
bool all_al16(std::initializer_list<const void *> ps) {
  for (const void *p : ps)
    if ((uintptr_t)p & 15) return false;
  return true;
}
bool all_al4(std::initializer_list<const void *> ps) {
  for (const void *p : ps)
    if ((uintptr_t)p & 3) return false;
  return true;
}

bool valid_dtype(int t) { return t == GLA_F32 || t == GLA_BF16; }

}  // namespace

namespace gla {

// The chunked forward after argument checks: plans (when the batch needs
// splitting) and launches. Shared by gla_fwd_chunked and gla_bwd_chunked.
gla_status fwd_core(const void *q, const void *k, const void *v, const float *g, const float *S0,
                    const int32_t *cu_seqlens, void *o, float *S_T, int B, int T, int H, int dk,
                    int dv, int N, int chunk_size, gla_dtype in_dtype, gla_dtype out_dtype,
                    void *workspace, size_t workspace_bytes, hipStream_t stream,
                    bool fixed_decay, bool rev, const DotOut *dot, bool f32_kernel,
                    int head_group, void *o2) {
  const bool has_cu = cu_seqlens != nullptr;
  FwdDims d;
  d.B = B;
  d.T = T;
  d.H = H;
  d.dk = dk;
  d.dv = dv;
  d.N = N;
  chunk_size = kernel_chunk(in_dtype, f32_kernel, chunk_size);
  d.C = chunk_size;
  d.gts = fixed_decay ? 0 : H / head_group;  // the gates have the real heads
  d.hg = head_group;
  d.o2 = o2;
  d.rev = rev;
  d.dot_x = dot ? static_cast<const uint16_t *>(dot->x) : nullptr;
  d.dot_part = dot ? dot->part : nullptr;
  d.dot_stride = dot ? dot->stride : 0;
  PlanLayout lay;
  const bool planned = make_plan(B, T, H, dk, dv, N, chunk_size, has_cu, cu_count(),
                                 f32_kernel ? GLA_F32 : in_dtype, lay);
  if (planned && (!workspace || workspace_bytes < lay.total_bytes)) return GLA_ERR_WORKSPACE;

  const bool bf = in_dtype == GLA_BF16, out_bf = out_dtype == GLA_BF16;
  auto run_chunks = [&](const WorkItem *items, const int *n_items, int grid_items, float *slots,
                        float *slot_gamma, bool state_pass) -> hipError_t {
    if (bf && !f32_kernel)
      return launch_chunk_bf16(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                               static_cast<const uint16_t *>(v), g, S0, S_T, o, out_bf, d, items,
                               n_items, grid_items, slots, slot_gamma, state_pass, stream);
    return launch_chunk_f32(q, k, v, g, S0, S_T, o, bf, out_bf, d, items, n_items, grid_items,
                            slots, slot_gamma, state_pass, stream);
  };

  hipError_t err;
  if (!planned) {
    err = run_chunks(nullptr, nullptr, B, nullptr, nullptr, false);
    return err == hipSuccess ? GLA_OK : GLA_ERR_HIP;
  }
  char *ws = static_cast<char *>(workspace);
  const PlanHeader *hdr = reinterpret_cast<const PlanHeader *>(ws + lay.off_header);
  const WorkItem *items = reinterpret_cast<const WorkItem *>(ws + lay.off_items);
  const WorkItem *sitems = reinterpret_cast<const WorkItem *>(ws + lay.off_state_items);
  float *slots = reinterpret_cast<float *>(ws + lay.off_slots);
  float *slot_gamma = reinterpret_cast<float *>(ws + lay.off_slot_gamma);
  // S_T over S0 (the one overlap the header allows): the last segment of a
  // split sequence writes S_T[seq] while its first segment, another
  // workgroup, reads S0[seq], so that one reads a copy made by the combine
  const bool s0_copy = S0 && S_T == S0;
  if ((err = launch_plan(cu_seqlens, d, lay, s0_copy, workspace, stream)) != hipSuccess)
    return GLA_ERR_HIP;
  if (lay.max_state_items > 0) {
    if ((err = run_chunks(sitems, &hdr->n_state_items, lay.max_state_items, slots, slot_gamma,
                          true)) != hipSuccess)
      return GLA_ERR_HIP;
    if ((err = launch_combine(S0, d, lay, s0_copy, workspace, stream)) != hipSuccess)
      return GLA_ERR_HIP;
  }
  err = run_chunks(items, &hdr->n_items, lay.max_items, slots, slot_gamma, false);
  return err == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

// Workspace of fwd_core for these sizes (0 when it runs without a plan).
size_t fwd_workspace(int B, int T, int H, int dk, int dv, int N, int chunk_size, bool has_cu,
                     gla_dtype in_dtype, bool f32_kernel) {
  PlanLayout lay;
  chunk_size = kernel_chunk(in_dtype, f32_kernel, chunk_size);
  if (!make_plan(B, T, H, dk, dv, N, chunk_size, has_cu, cu_count(),
                 f32_kernel ? GLA_F32 : in_dtype, lay))
    return 0;
  return lay.total_bytes;
}

}  // namespace gla

extern "C" {

const char *gla_status_string(gla_status s) {
  switch (s) {
    case GLA_OK: return "GLA_OK";
    case GLA_ERR_INVALID_ARGUMENT: return "GLA_ERR_INVALID_ARGUMENT";
    case GLA_ERR_UNSUPPORTED: return "GLA_ERR_UNSUPPORTED";
    case GLA_ERR_WORKSPACE: return "GLA_ERR_WORKSPACE";
    case GLA_ERR_HIP: return "GLA_ERR_HIP";
  }
  return "GLA_UNKNOWN_STATUS";
}

size_t gla_fwd_chunked_workspace_size(int B, int T, int H, int dk, int dv, int num_seqs,
                                      int chunk_size, int has_cu_seqlens, gla_dtype in_dtype) {
  if (B < 0 || T < 0 || H <= 0 || num_seqs < 0 || !fwd_dims(dk, dv) ||
      !supported_chunk(chunk_size) || !valid_dtype(in_dtype))
    return 0;
  return fwd_workspace(B, T, H, dk, dv, num_seqs, chunk_size, has_cu_seqlens != 0, in_dtype);
}

}  // extern "C"

namespace {

// Argument checks of the forward entry points (GLA_OK: valid).
gla_status fwd_validate(const void *q, const void *k, const void *v, const float *g,
                        const float *S0, const int32_t *cu_seqlens, void *o, float *S_T, int B,
                        int T, int H, int dk, int dv, int num_seqs, int chunk_size,
                        gla_dtype in_dtype, gla_dtype out_dtype, const void *workspace,
                        bool fixed_decay) {
  if (B < 0 || T < 0 || H < 0 || num_seqs < 0) return GLA_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return GLA_ERR_INVALID_ARGUMENT;
  const bool has_cu = cu_seqlens != nullptr;
  if (has_cu ? (B != 1) : (num_seqs != B)) return GLA_ERR_INVALID_ARGUMENT;
  if ((long)B * T > INT_MAX) return GLA_ERR_INVALID_ARGUMENT;
  if (!fwd_dims(dk, dv)) return GLA_ERR_UNSUPPORTED;
  if (!supported_chunk(chunk_size)) return GLA_ERR_UNSUPPORTED;
  if (!all_al16({q, k, v, o, S0, S_T, workspace}) || !all_al4({g, cu_seqlens}))
    return GLA_ERR_INVALID_ARGUMENT;
  const int N = num_seqs;
  if (H == 0 || N == 0) return GLA_OK;
  const size_t ntok = (size_t)B * T * H;
  const size_t es = dtype_size(in_dtype);
  const size_t bytes_qk = ntok * dk * es, bytes_v = ntok * dv * es;
  const size_t bytes_g = fixed_decay ? (size_t)H * 4 : ntok * 4;
  const size_t bytes_o = ntok * dv * dtype_size(out_dtype);
  const size_t bytes_S = (size_t)N * H * dk * dv * 4;
  if (ntok > 0 && (!q || !k || !v || !g || !o)) return GLA_ERR_INVALID_ARGUMENT;
  if (overlaps(o, bytes_o, q, bytes_qk) || overlaps(o, bytes_o, k, bytes_qk) ||
      overlaps(o, bytes_o, v, bytes_v) || overlaps(o, bytes_o, g, bytes_g) ||
      overlaps(o, bytes_o, S0, S0 ? bytes_S : 0) || overlaps(o, bytes_o, S_T, S_T ? bytes_S : 0))
    return GLA_ERR_INVALID_ARGUMENT;
  if (S_T && S_T != S0 &&
      (overlaps(S_T, bytes_S, S0, S0 ? bytes_S : 0) || overlaps(S_T, bytes_S, q, bytes_qk) ||
       overlaps(S_T, bytes_S, k, bytes_qk) || overlaps(S_T, bytes_S, v, bytes_v) ||
       overlaps(S_T, bytes_S, g, bytes_g)))
    return GLA_ERR_INVALID_ARGUMENT;
  return GLA_OK;
}

// Argument checks, then the forward.
gla_status fwd_checked(const void *q, const void *k, const void *v, const float *g,
                       const float *S0, const int32_t *cu_seqlens, void *o, float *S_T, int B,
                       int T, int H, int dk, int dv, int num_seqs, int chunk_size,
                       gla_dtype in_dtype, gla_dtype out_dtype, void *workspace,
                       size_t workspace_bytes, void *stream_, bool fixed_decay) {
  const gla_status st = fwd_validate(q, k, v, g, S0, cu_seqlens, o, S_T, B, T, H, dk, dv,
                                     num_seqs, chunk_size, in_dtype, out_dtype, workspace,
                                     fixed_decay);
  if (st != GLA_OK || H == 0 || num_seqs == 0) return st;
  return gla::fwd_core(q, k, v, g, S0, cu_seqlens, o, S_T, B, T, H, dk, dv, num_seqs,
                       chunk_size, in_dtype, out_dtype, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream_), fixed_decay);
}

}  // namespace

extern "C" {

gla_status gla_fwd_chunked(const void *q, const void *k, const void *v, const float *g,
                           const float *S0, const int32_t *cu_seqlens, void *o, float *S_T,
                           int B, int T, int H, int dk, int dv, int num_seqs, int chunk_size,
                           gla_dtype in_dtype, gla_dtype out_dtype, void *workspace,
                           size_t workspace_bytes, void *stream) {
  return fwd_checked(q, k, v, g, S0, cu_seqlens, o, S_T, B, T, H, dk, dv, num_seqs, chunk_size,
                     in_dtype, out_dtype, workspace, workspace_bytes, stream, false);
}

}  // extern "C"

// Scratch of gla_fwd_chunked_noalloc: one fixed array per GPU, held by the
// loaded library until the process ends. Host code never uses the array's
// name as an address: each device's address comes from hipGetSymbolAddress
// once, with that device current, and is kept per device.
static constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, or nullptr if it cannot be had.
void *scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);  // racing threads store the same
  }
  return p;
}

}  // namespace

extern "C" {

size_t gla_fwd_chunked_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

gla_status gla_fwd_chunked_noalloc(const void *q, const void *k, const void *v, const float *g,
                                   const float *S0, const int32_t *cu_seqlens, void *o,
                                   float *S_T, int B, int T, int H, int dk, int dv,
                                   int num_seqs, int chunk_size, gla_dtype in_dtype,
                                   gla_dtype out_dtype, void *stream) {
  // the checks of gla_fwd_chunked (no workspace to check), then the scratch
  gla_status st = fwd_validate(q, k, v, g, S0, cu_seqlens, o, S_T, B, T, H, dk, dv, num_seqs,
                               chunk_size, in_dtype, out_dtype, nullptr, false);
  if (st != GLA_OK || H == 0 || num_seqs == 0) return st;
  const size_t need =
      fwd_workspace(B, T, H, dk, dv, num_seqs, chunk_size, cu_seqlens != nullptr, in_dtype);
  if (need > kNoAllocScratchBytes) return GLA_ERR_WORKSPACE;
  void *ws = nullptr;
  if (need > 0 && !(ws = scratch_ptr())) return GLA_ERR_HIP;
  return gla::fwd_core(q, k, v, g, S0, cu_seqlens, o, S_T, B, T, H, dk, dv, num_seqs,
                       chunk_size, in_dtype, out_dtype, ws, need, static_cast<hipStream_t>(stream),
                       false);
}

gla_status gla_fwd_chunked_fixed_decay(const void *q, const void *k, const void *v,
                                       const float *log_lambda, const float *S0,
                                       const int32_t *cu_seqlens, void *o, float *S_T, int B,
                                       int T, int H, int dk, int dv, int num_seqs,
                                       int chunk_size, gla_dtype in_dtype, gla_dtype out_dtype,
                                       void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_checked(q, k, v, log_lambda, S0, cu_seqlens, o, S_T, B, T, H, dk, dv, num_seqs,
                     chunk_size, in_dtype, out_dtype, workspace, workspace_bytes, stream, true);
}

}  // extern "C"

namespace {

// Head shapes of the backward: (d_k, d_v) in {64, 128}^2 on the forward
// kernels of the input type, and the Laplace 96 x 192 heads, whose dq and dk
// runs are forwards with 192-dim keys: with bf16 inputs those run as two
// 96-dim key halves (bwd_split_keys below), with fp32 inputs on the fp32
// kernel, the dv run with them.
bool bwd_dims(int dk, int dv) {
  return (supported_head_dim(dk) && supported_head_dim(dv)) || (dk == 96 && dv == 192);
}
bool bwd_f32_kernel(int dk, int dv) { return dk == 96 && dv == 192; }
// The dv run of those heads is a 96 x 192 forward: on the twelve-wavefront
// bf16 kernel for bf16 inputs at chunk 64, otherwise with the dq and dk runs.
bool bwd_dv_f32_kernel(int dk, int dv, int C, gla_dtype in_dtype) {
  (void)C;  // the bf16 kernels run every chunk size as 64-token chunks
  return bwd_f32_kernel(dk, dv) && in_dtype != GLA_BF16;
}

// bf16 inputs with 96 x 192 heads: the dq and dk runs (192-dim keys, 96-dim
// values) run on the twelve-wavefront kernel as two 96-dim key halves, head
// groups of two, whose outputs add.
bool bwd_split_keys(int dk, int dv, gla_dtype in_dtype) {
  return dk == 96 && dv == 192 && in_dtype == GLA_BF16;
}

// Workspace layout of the backward (all offsets 256-byte aligned).
struct BwdLayout {
  size_t s0t, dstt, stt, a0, dqp, dkp, dq2, dk2, fws, total, fws_bytes;
  bool fused_dots;  // dq and dk passes write partial q.dq, k.dk (bf16, chunk 64)
  bool split;       // dq, dk runs in two key halves (dq2, dk2: the second halves)
};

BwdLayout bwd_layout(int B, int T, int H, int dk, int dv, int N, int C, bool has_cu,
                     gla_dtype in_dtype) {
  BwdLayout L;
  const size_t ntok = (size_t)B * T * H, es = dtype_size(in_dtype);
  const size_t mat = (size_t)N * H * dk * dv * 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  (void)es;
  L.s0t = take(mat);
  L.dstt = take(mat);
  L.stt = take(mat);
  L.a0 = take(mat);
  const bool f32k = bwd_f32_kernel(dk, dv);
  L.split = bwd_split_keys(dk, dv, in_dtype);
  L.fused_dots = in_dtype == GLA_BF16 && !f32k;  // the 64-token kernel's row dots
  const size_t parts = L.fused_dots ? (size_t)(dk / 16) * ntok * 4 : 0;
  L.dqp = take(parts);
  L.dkp = take(parts);
  L.dq2 = take(L.split ? ntok * dk * 4 : 0);
  L.dk2 = take(L.split ? ntok * dk * 4 : 0);
  const size_t f1 = L.split ? fwd_workspace(B, T, 2 * H, dk, dk, N, C, has_cu, in_dtype, false)
                            : fwd_workspace(B, T, H, dv, dk, N, C, has_cu, in_dtype, f32k);
  const size_t f2 = fwd_workspace(B, T, H, dk, dv, N, C, has_cu, in_dtype,
                                  bwd_dv_f32_kernel(dk, dv, C, in_dtype));
  L.fws_bytes = f1 > f2 ? f1 : f2;
  L.fws = take(L.fws_bytes);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t gla_bwd_chunked_workspace_size(int B, int T, int H, int dk, int dv, int num_seqs,
                                      int chunk_size, int has_cu_seqlens, gla_dtype in_dtype) {
  if (B < 0 || T < 0 || H <= 0 || num_seqs < 0 || !bwd_dims(dk, dv) ||
      !supported_chunk(chunk_size) || !valid_dtype(in_dtype))
    return 0;
  return bwd_layout(B, T, H, dk, dv, num_seqs, chunk_size, has_cu_seqlens != 0, in_dtype).total;
}

gla_status gla_bwd_chunked(const void *q, const void *k, const void *v, const float *g,
                           const float *S0, const int32_t *cu_seqlens, const void *dO,
                           const float *dS_T, float *dq, float *dk, float *dv, float *dg,
                           float *dS0, int B, int T, int H, int dk_dim, int dv_dim, int num_seqs,
                           int chunk_size, gla_dtype in_dtype, void *workspace,
                           size_t workspace_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int DK = dk_dim, DV = dv_dim;
  if (B < 0 || T < 0 || H < 0 || num_seqs < 0) return GLA_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(in_dtype)) return GLA_ERR_INVALID_ARGUMENT;
  const bool has_cu = cu_seqlens != nullptr;
  if (has_cu ? (B != 1) : (num_seqs != B)) return GLA_ERR_INVALID_ARGUMENT;
  if ((long)B * T > INT_MAX) return GLA_ERR_INVALID_ARGUMENT;
  if (!bwd_dims(DK, DV)) return GLA_ERR_UNSUPPORTED;
  if (!supported_chunk(chunk_size)) return GLA_ERR_UNSUPPORTED;
  if (!all_al16({q, k, v, dO, S0, dS_T, dq, dk, dv, dS0, workspace}) ||
      !all_al4({g, dg, cu_seqlens}))
    return GLA_ERR_INVALID_ARGUMENT;
  const int N = num_seqs;
  if (H == 0 || N == 0) return GLA_OK;
  const size_t ntok = (size_t)B * T * H;
  const size_t es = dtype_size(in_dtype);
  const size_t b_qk = ntok * DK * es, b_v = ntok * DV * es, b_g = ntok * 4;
  const size_t b_dqk = ntok * DK * 4, b_dv = ntok * DV * 4;
  const size_t b_S = (size_t)N * H * DK * DV * 4;
  if (ntok > 0 && (!q || !k || !v || !g || !dO || !dq || !dk || !dv || !dg))
    return GLA_ERR_INVALID_ARGUMENT;
  struct Buf {
    const void *p;
    size_t n;
  };
  const Buf ins[] = {{q, b_qk}, {k, b_qk}, {v, b_v}, {g, b_g}, {dO, b_v},
                     {S0, S0 ? b_S : 0}, {dS_T, dS_T ? b_S : 0}};
  const Buf outs[] = {{dq, b_dqk}, {dk, b_dqk}, {dv, b_dv}, {dg, b_g}, {dS0, dS0 ? b_S : 0}};
  for (const Buf &o : outs) {
    for (const Buf &i : ins)
      if (overlaps(o.p, o.n, i.p, i.n)) return GLA_ERR_INVALID_ARGUMENT;
    for (const Buf &o2 : outs)
      if (&o2 != &o && overlaps(o.p, o.n, o2.p, o2.n)) return GLA_ERR_INVALID_ARGUMENT;
  }
  const BwdLayout L = bwd_layout(B, T, H, DK, DV, N, chunk_size, has_cu, in_dtype);
  if (!workspace || workspace_bytes < L.total) return GLA_ERR_WORKSPACE;

  char *ws = static_cast<char *>(workspace);
  float *s0t = S0 ? reinterpret_cast<float *>(ws + L.s0t) : nullptr;
  float *dstt = dS_T ? reinterpret_cast<float *>(ws + L.dstt) : nullptr;
  float *stt = reinterpret_cast<float *>(ws + L.stt);
  float *a0 = reinterpret_cast<float *>(ws + L.a0);
  void *fws = L.fws_bytes ? ws + L.fws : nullptr;
  // with the chunk-64 bf16 kernels the dq and dk runs also write the partial
  // sums of q.dq and k.dk (one per 16-column group) for the gate gradient
  const DotOut dq_dot{q, reinterpret_cast<float *>(ws + L.dqp), (long)B * T};
  const DotOut dk_dot{k, reinterpret_cast<float *>(ws + L.dkp), (long)B * T};
  const bool fuse = L.fused_dots;
  const bool f32k = bwd_f32_kernel(DK, DV) && !L.split;
  float *dq2 = L.split ? reinterpret_cast<float *>(ws + L.dq2) : nullptr;
  float *dk2 = L.split ? reinterpret_cast<float *>(ws + L.dk2) : nullptr;
  // transposed initial states
  if ((S0 && launch_transpose(S0, s0t, N * H, DK, DV, stream) != hipSuccess) ||
      (dS_T && launch_transpose(dS_T, dstt, N * H, DK, DV, stream) != hipSuccess))
    return GLA_ERR_HIP;
  gla_status st;
  // dq: forward with (q, k, v) = (dO, v, k) on the transposed state; its final
  // state is S_T^T
  if (L.split)  // 192-dim keys as two 96-dim halves: heads of [.., 2, 96], states [2, 96, 96]
    st = fwd_core(dO, v, k, g, s0t, cu_seqlens, dq, stt, B, T, 2 * H, DK, DK, N, chunk_size,
                  in_dtype, GLA_F32, fws, L.fws_bytes, stream, false, false, nullptr, false, 2,
                  dq2);
  else
    st = fwd_core(dO, v, k, g, s0t, cu_seqlens, dq, stt, B, T, H, DV, DK, N, chunk_size,
                  in_dtype, GLA_F32, fws, L.fws_bytes, stream, false, false,
                  fuse ? &dq_dot : nullptr, f32k);
  if (st != GLA_OK) return st;
  // dv: the reversed-time run with (q, k, v) = (k, q, dO) from dS_T; ends in A_0
  st = fwd_core(k, q, dO, g, dS_T, cu_seqlens, dv, a0, B, T, H, DK, DV, N, chunk_size, in_dtype,
                GLA_F32, fws, L.fws_bytes, stream, false, true, nullptr,
                bwd_dv_f32_kernel(DK, DV, chunk_size, in_dtype));
  if (st != GLA_OK) return st;
  // dk: the reversed-time run with (q, k, v) = (v, dO, q) from dS_T^T
  if (L.split)
    st = fwd_core(v, dO, q, g, dstt, cu_seqlens, dk, nullptr, B, T, 2 * H, DK, DK, N, chunk_size,
                  in_dtype, GLA_F32, fws, L.fws_bytes, stream, false, true, nullptr, false, 2,
                  dk2);
  else
    st = fwd_core(v, dO, q, g, dstt, cu_seqlens, dk, nullptr, B, T, H, DV, DK, N, chunk_size,
                  in_dtype, GLA_F32, fws, L.fws_bytes, stream, false, true,
                  fuse ? &dk_dot : nullptr, f32k);
  if (st != GLA_OK) return st;
  if (launch_dgate(q, k, dq, dk, g, stt, dstt, a0, dg, dS0, cu_seqlens, N, T, H, DK, DV,
                   in_dtype == GLA_BF16, fuse ? dq_dot.part : nullptr,
                   fuse ? dk_dot.part : nullptr, fuse ? DK / 16 : 0, stream, dq2,
                   dk2) != hipSuccess)
    return GLA_ERR_HIP;
  return GLA_OK;
}

gla_status gla_decode_step(const void *q, const void *k, const void *v, const float *g,
                           float *S, void *o, int N, int H, int dk, int dv, gla_dtype in_dtype,
                           gla_dtype out_dtype, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (N < 0 || H < 0) return GLA_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return GLA_ERR_INVALID_ARGUMENT;
  if (!fwd_dims(dk, dv)) return GLA_ERR_UNSUPPORTED;
  if (!all_al16({q, k, v, S, o}) || !all_al4({g})) return GLA_ERR_INVALID_ARGUMENT;
  const size_t pairs = (size_t)N * H;
  if (pairs == 0) return GLA_OK;
  if (pairs > (size_t)INT_MAX) return GLA_ERR_INVALID_ARGUMENT;
  if (!q || !k || !v || !g || !S || !o) return GLA_ERR_INVALID_ARGUMENT;
  const size_t es = dtype_size(in_dtype);
  const size_t bq = pairs * dk * es, bv = pairs * dv * es, bg = pairs * 4;
  const size_t bS = pairs * dk * dv * 4, bo = pairs * dv * dtype_size(out_dtype);
  if (overlaps(o, bo, q, bq) || overlaps(o, bo, k, bq) || overlaps(o, bo, v, bv) ||
      overlaps(o, bo, g, bg) || overlaps(o, bo, S, bS) || overlaps(S, bS, q, bq) ||
      overlaps(S, bS, k, bq) || overlaps(S, bS, v, bv) || overlaps(S, bS, g, bg))
    return GLA_ERR_INVALID_ARGUMENT;
  const hipError_t err = launch_decode(q, k, v, g, S, o, N, H, dk, dv, in_dtype == GLA_BF16,
                                       out_dtype == GLA_BF16, nullptr, nullptr, 0, cu_count(),
                                       stream);
  return err == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

gla_status gla_decode_slot_order(const int32_t *slots, int N, int P, size_t slot_bytes,
                                 int32_t *order, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (N < 0 || P < 0) return GLA_ERR_INVALID_ARGUMENT;
  if (P > kMaxOrderPool) return GLA_ERR_UNSUPPORTED;
  if (N == 0) return GLA_OK;
  if (!slots || !order || !all_al4({slots, order})) return GLA_ERR_INVALID_ARGUMENT;
  if (overlaps(order, (size_t)N * 8, slots, (size_t)N * 4)) return GLA_ERR_INVALID_ARGUMENT;
  // entries above 4 MiB form no blocks (slot order); the clamp keeps the size a long
  const long sb = slot_bytes > ((size_t)1 << 40) ? 0 : (long)slot_bytes;
  return launch_slot_order(slots, N, P, sb, order, stream) == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

gla_status gla_decode_step_slots(const void *q, const void *k, const void *v, const float *g,
                                 float *S_pool, const int32_t *slots, const int32_t *order,
                                 void *o, int N, int P, int H, int dk, int dv, gla_dtype in_dtype,
                                 gla_dtype out_dtype, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (N < 0 || P < 0 || H < 0) return GLA_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return GLA_ERR_INVALID_ARGUMENT;
  if (!fwd_dims(dk, dv)) return GLA_ERR_UNSUPPORTED;
  if (!all_al16({q, k, v, S_pool, o}) || !all_al4({g, slots, order}))
    return GLA_ERR_INVALID_ARGUMENT;
  const size_t pairs = (size_t)N * H;
  if (pairs == 0) return GLA_OK;
  if (pairs > (size_t)INT_MAX || (size_t)P * H > (size_t)INT_MAX) return GLA_ERR_INVALID_ARGUMENT;
  if (!q || !k || !v || !g || !slots || !o || (P > 0 && !S_pool)) return GLA_ERR_INVALID_ARGUMENT;
  const size_t es = dtype_size(in_dtype);
  const size_t bq = pairs * dk * es, bv = pairs * dv * es, bg = pairs * 4, bs = (size_t)N * 4;
  const size_t bS = (size_t)P * H * dk * dv * 4, bo = pairs * dv * dtype_size(out_dtype);
  if (overlaps(o, bo, q, bq) || overlaps(o, bo, k, bq) || overlaps(o, bo, v, bv) ||
      overlaps(o, bo, g, bg) || overlaps(o, bo, S_pool, bS) || overlaps(o, bo, slots, bs) ||
      overlaps(S_pool, bS, q, bq) || overlaps(S_pool, bS, k, bq) || overlaps(S_pool, bS, v, bv) ||
      overlaps(S_pool, bS, g, bg) || overlaps(S_pool, bS, slots, bs) ||
      overlaps(o, bo, order, order ? 2 * bs : 0) || overlaps(S_pool, bS, order, order ? 2 * bs : 0))
    return GLA_ERR_INVALID_ARGUMENT;
  const hipError_t err = launch_decode(q, k, v, g, S_pool, o, N, H, dk, dv, in_dtype == GLA_BF16,
                                       out_dtype == GLA_BF16, slots, order, P, cu_count(), stream);
  return err == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

gla_status gla_mixer_epilogue(const void *o, const void *q, const void *k, const void *v,
                              const void *g, const float *a, const float *rms_w, float eps,
                              void *z, int n_tokens, int H, int dk, int dv, gla_dtype o_dtype,
                              gla_dtype in_dtype, gla_dtype out_dtype, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (n_tokens < 0 || H < 0) return GLA_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(o_dtype) || !valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return GLA_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.f) || eps > 3.4e38f) return GLA_ERR_INVALID_ARGUMENT;  // NaN, negative, inf
  if (!fwd_dims(dk, dv)) return GLA_ERR_UNSUPPORTED;
  if (!all_al16({o, q, k, v, g, a, rms_w, z})) return GLA_ERR_INVALID_ARGUMENT;
  const size_t rows = (size_t)n_tokens * H;
  if (rows == 0) return GLA_OK;
  if (rows > (size_t)INT_MAX) return GLA_ERR_INVALID_ARGUMENT;
  if (!o || !q || !k || !v || !g || !a || !rms_w || !z) return GLA_ERR_INVALID_ARGUMENT;
  const size_t es = dtype_size(in_dtype);
  const size_t bo = rows * dv * dtype_size(o_dtype), bqk = rows * dk * es, bv = rows * dv * es;
  const size_t ba = (size_t)H * dk * 4, bw = (size_t)H * dv * 4;
  const size_t bz = rows * dv * dtype_size(out_dtype);
  const bool in_place = z == o && o_dtype == out_dtype;
  if ((!in_place && overlaps(z, bz, o, bo)) || overlaps(z, bz, q, bqk) ||
      overlaps(z, bz, k, bqk) || overlaps(z, bz, v, bv) || overlaps(z, bz, g, bv) ||
      overlaps(z, bz, a, ba) || overlaps(z, bz, rms_w, bw))
    return GLA_ERR_INVALID_ARGUMENT;
  const hipError_t err =
      launch_mixer_epilogue(o, q, k, v, g, a, rms_w, eps, z, (long)rows, H, dk, dv,
                            o_dtype == GLA_BF16, in_dtype == GLA_BF16, out_dtype == GLA_BF16,
                            stream);
  return err == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

gla_status gla_decode_mixer(const void *q, const void *k, const void *v, const float *g,
                            float *S, const int32_t *slots, const int32_t *order, int P,
                            const void *g_out,
                            const float *a, const float *rms_w, float eps, void *z, int N, int H,
                            int dk, int dv, gla_dtype in_dtype, gla_dtype out_dtype,
                            void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (N < 0 || H < 0 || (slots && P < 0)) return GLA_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return GLA_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.f) || eps > 3.4e38f) return GLA_ERR_INVALID_ARGUMENT;
  if (!fwd_dims(dk, dv)) return GLA_ERR_UNSUPPORTED;
  if (order && !slots) return GLA_ERR_INVALID_ARGUMENT;
  if (!all_al16({q, k, v, S, g_out, a, rms_w, z}) || !all_al4({g, slots, order}))
    return GLA_ERR_INVALID_ARGUMENT;
  const size_t pairs = (size_t)N * H;
  if (pairs == 0) return GLA_OK;
  const size_t n_states = slots ? (size_t)P * H : pairs;
  if (pairs > (size_t)INT_MAX || n_states > (size_t)INT_MAX) return GLA_ERR_INVALID_ARGUMENT;
  if (!q || !k || !v || !g || !g_out || !a || !rms_w || !z || (n_states > 0 && !S))
    return GLA_ERR_INVALID_ARGUMENT;
  const size_t es = dtype_size(in_dtype);
  const size_t bq = pairs * dk * es, bv = pairs * dv * es, bg = pairs * 4;
  const size_t bS = n_states * dk * dv * 4, bz = pairs * dv * dtype_size(out_dtype);
  const size_t ba = (size_t)H * dk * 4, bw = (size_t)H * dv * 4, bs = slots ? (size_t)N * 4 : 0;
  const void *ins[] = {q, k, v, g, g_out, a, rms_w, slots, order};
  const size_t nins[] = {bq, bq, bv, bg, bv, ba, bw, bs, order ? 2 * bs : 0};
  for (int i = 0; i < 9; ++i)
    if (overlaps(z, bz, ins[i], nins[i]) || overlaps(S, bS, ins[i], nins[i]))
      return GLA_ERR_INVALID_ARGUMENT;
  if (overlaps(z, bz, S, bS)) return GLA_ERR_INVALID_ARGUMENT;
  MixerArgs m{q, k, v, g, S, g_out, a, rms_w, eps, z, slots, slots ? P : 0, H, (long)pairs,
              ReqMap{order, N, 1, 0, 1}};
  const hipError_t err =
      launch_decode_mixer(m, dk, dv, in_dtype == GLA_BF16, out_dtype == GLA_BF16, stream);
  return err == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

}  // extern "C"
