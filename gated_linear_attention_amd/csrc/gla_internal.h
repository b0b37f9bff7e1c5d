// Host/device interfaces between the C ABI layer and the GLA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gla.h"
#include "plan_host.h"

namespace gla {

// dims of the flattened problem
struct FwdDims {
  int B, T, H, dk, dv, N, C;
  int gts;  // gate token stride in floats: H (log_g [.., T, H]) or 0 (one fixed log-decay per head)
  // time-reversed run: logical token t of sequence [sb, se) is memory row
  // sb + se - 1 - t for q, k, v and o, and its gate is log_g[se - (t - sb)]
  // (0 at t = sb): the adjoint recurrence of the backward
  bool rev;
  // optional row dot products of the outputs with x ([.., T, H, dv] bf16):
  // part[(p * H + h) * stride + token] = sum over the columns of column group
  // p of o * x (stride = tokens; the backward's q . dq and k . dk); chunk 64,
  // bf16 only
  const uint16_t *dot_x;
  float *dot_part;
  long dot_stride;
  // head groups (bf16 kernel only): H counts the heads of q, k and the states;
  // v, the gates and the outputs have H / hg heads, and heads with h % hg != 0
  // write their outputs to o2 (see chunk_bf16_w8_kernel)
  int hg = 1;
  void *o2 = nullptr;
};

// Row dot products requested from a forward run (see FwdDims::dot_x).
struct DotOut {
  const void *x;
  float *part;
  long stride;
};

// slots == nullptr: state of pair (n, h) is S[n, h]; otherwise S[slots[n], h]
// for slots[n] in [0, P), and a padded lane (no state touched, o = 0) else.
// Batches with fewer than two (sequence, head) pairs per CU (n_cu CUs) split
// each pair's columns over several workgroups.
// Launch position -> request of the decode kernels (decode.hip): order[j]
// when the caller passed gla_decode_slot_order's order (order [2, n]: the
// requests, then their slots), else groups of gs requests with group g at position
// (g * stride) % ng (requests past ng * gs in place).
struct ReqMap {
  const int32_t *order;
  int n, gs, ng, stride;
  __device__ __forceinline__ int operator()(int j) const {  // -1: not a request
    if (order) {
      const int r = order[j];
      return r >= 0 && r < n ? r : -1;
    }
    if (j >= gs * ng) return j;
    const int g = j / gs;
    return gs * (int)(((long)g * stride) % ng) + (j - g * gs);
  }
  // the pool slot of position j (request r): from the order's second row, a
  // load that does not wait for the first
  __device__ __forceinline__ int slot(int j, const int32_t *slots, int r) const {
    return order ? order[n + j] : slots[r];
  }
};
ReqMap make_req_map(const int32_t *order, int n, long bytes_per_request);

// The largest pool gla_decode_slot_order sorts (one LDS counter per entry).
constexpr int kMaxOrderPool = 32768;
hipError_t launch_slot_order(const int32_t *slots, int N, int P, long slot_bytes, int32_t *order,
                             hipStream_t stream);

// order: the pool-order request order (with slots only), or null.
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g, float *S,
                         void *o, int N, int H, int dk, int dv, bool in_bf16, bool out_bf16,
                         const int32_t *slots, const int32_t *order, int P, int n_cu,
                         hipStream_t stream);

// s0_copy: the output pass writes S_T over S0, so the first segment of a
// split sequence reads a copy of S0 that the combine leaves in the chain's
// first slot (another workgroup writes S_T[seq]).
hipError_t launch_plan(const int32_t *cu_seqlens, const FwdDims &d, const PlanLayout &lay,
                       bool s0_copy, void *workspace, hipStream_t stream);

hipError_t launch_combine(const float *S0, const FwdDims &d, const PlanLayout &lay,
                          bool s0_copy, void *workspace, hipStream_t stream);

// fp32 arithmetic on fp32 inputs, or on bf16 inputs (in_bf16; d_k 96 or 192,
// fp32 o: the backward's runs for the 96 x 192 heads). state_pass: compute
// segment-local states only.
hipError_t launch_chunk_f32(const void *q, const void *k, const void *v, const float *g,
                            const float *S0, float *S_T, void *o, bool in_bf16, bool out_bf16,
                            const FwdDims &d, const WorkItem *items, const int *n_items,
                            int grid_items, float *slots, float *slot_gamma, bool state_pass,
                            hipStream_t stream);

// bf16 inputs on the matrix cores, fp32 accumulation and state: the eight-
// (twelve-) wavefront kernel of chunk_bf16_w8.hip, 64-token chunks (d.C = 64).
hipError_t launch_chunk_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const float *g, const float *S0, float *S_T, void *o, bool out_bf16,
                             const FwdDims &d, const WorkItem *items, const int *n_items,
                             int grid_items, float *slots, float *slot_gamma, bool state_pass,
                             hipStream_t stream);

// The output pass for 128-dim keys on the wavefront-specialised kernel of
// chunk_bf16_ws.hip (d.C = 64, d.dv a multiple of 64, no head groups;
// reversed and dot-product runs with per-token gates and fp32 outputs);
// launch_chunk_bf16 routes there.
hipError_t launch_chunk_bf16_ws(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const float *g, const float *S0, float *S_T, void *o,
                                bool out_bf16, const FwdDims &d, const WorkItem *items,
                                const int *n_items, int grid_items, const float *slots,
                                hipStream_t stream);
// The state pass (split sequences' pieces) for 128-dim keys on the same layout.
hipError_t launch_chunk_bf16_ws_state(const uint16_t *k, const uint16_t *v, const float *g,
                                      const FwdDims &d, const WorkItem *items, const int *n_items,
                                      int grid_items, float *slots, float *slot_gamma,
                                      hipStream_t stream);

// The chunked forward after argument checks (gla_api.hip), and its workspace.
// g is log_g [.., T, H], or with fixed_decay one log-decay per head [H]. rev
// runs every sequence in reversed time (FwdDims::rev): o is written in the
// inputs' order, S0 / S_T are the reversed run's initial and final states.
gla_status fwd_core(const void *q, const void *k, const void *v, const float *g, const float *S0,
                    const int32_t *cu_seqlens, void *o, float *S_T, int B, int T, int H, int dk,
                    int dv, int N, int chunk_size, gla_dtype in_dtype, gla_dtype out_dtype,
                    void *workspace, size_t workspace_bytes, hipStream_t stream,
                    bool fixed_decay = false, bool rev = false, const DotOut *dot = nullptr,
                    bool f32_kernel = false, int head_group = 1, void *o2 = nullptr);
// f32_kernel: run the fp32 kernel whatever in_dtype is (its workspace plan differs).
size_t fwd_workspace(int B, int T, int H, int dk, int dv, int N, int chunk_size, bool has_cu,
                     gla_dtype in_dtype, bool f32_kernel = false);
// Backward helpers (bwd.hip).
hipError_t launch_transpose(const float *in, float *out, int count, int rows, int cols,
                            hipStream_t stream);
// The gate gradient dl (reverse cumulative sums of q.dq - k.dk per sequence)
// and dS0. With n_part > 0 the dots come from the forward runs' partial sums
// dq_part / dk_part; otherwise they are formed from q, dq, k, dk first.
// With dq2 / dk2 (the second key halves of a split-key run: head groups of
// two, see FwdDims::hg), dq += dq2 and dk += dk2 first, in the same pass as
// the dots.
hipError_t launch_dgate(const void *q, const void *k, float *dq, float *dk, const float *lg,
                        const float *ST_t, const float *dST_t, const float *A0, float *dl,
                        float *dS0, const int32_t *cu, int N, int T, int H, int DK, int DV,
                        bool in_bf16, const float *dq_part, const float *dk_part, int n_part,
                        hipStream_t stream, const float *dq2 = nullptr,
                        const float *dk2 = nullptr);

// One decode step with the mixer epilogue fused (decode.hip): S (or the pool
// entries slots[n], as launch_decode) updated in place, z written; o is not.
struct MixerArgs {
  const void *q, *k, *v;
  const float *g;
  float *S;
  const void *gout;
  const float *a, *w;
  float eps;
  void *z;
  const int32_t *slots;
  int P, H;
  long pairs;
  ReqMap map;  // map.order: gla_decode_slot_order's request order, or null
};
hipError_t launch_decode_mixer(const MixerArgs &m, int dk, int dv, bool in_bf16, bool out_bf16,
                               hipStream_t stream);

// Token-mixer epilogue (epilogue.hip): n_rows = tokens x heads rows.
hipError_t launch_mixer_epilogue(const void *o, const void *q, const void *k, const void *v,
                                 const void *g, const float *a, const float *w, float eps,
                                 void *z, long n_rows, int H, int dk, int dv, bool o_bf16,
                                 bool in_bf16, bool out_bf16, hipStream_t stream);

}  // namespace gla
