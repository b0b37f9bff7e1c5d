// Varlen / long-sequence work planning for the chunked forward, on the device.
//
// The scheduler turns cu_seqlens (read on the GPU, so the host never waits
// for it) into work items, each one run of at most `seg_len` tokens of one
// sequence. Items are ordered longest first (a counting sort on their chunk
// count) so the workgroup dispatcher's greedy placement balances sequences
// of very different lengths. A sequence longer than seg_len is split into
// segments: a state pass computes the local state and total log-decay of
// every non-last segment, in n_sub pieces of sub_len tokens (so that the pass
// has enough workgroups to fill the GPU), the combine kernel chains them into
// every segment's start state, and the output pass then runs all segments in
// parallel. The chain
// uses that the per-token update is affine in S, so whole segments compose:
// the state after a segment is exp(sum of its log-gates) times the state
// before it plus the segment's own contribution from a zero state (Laplace 3B
// on AWS Trainium2, "Challenge 1": the state advances by the decay compounded
// over a chunk; a segment is a run of chunks).
#include <algorithm>

#include "gla_common.h"
#include "gla_internal.h"

namespace gla {

// Exclusive scan of one int across a 1024-thread block; returns the block total.
__device__ int block_exclusive_scan_1024(int x, int *scratch /* >= 16 ints */, int &total) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off *= 2) {
    int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      int t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[16] = run;
  }
  __syncthreads();
  const int excl = scratch[wave] + incl - x;
  total = scratch[16];
  __syncthreads();
  return excl;
}

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t *__restrict__ cu, int N, int T,
                                                    int L, int C, int Ls, int n_sub,
                                                    int max_items,
                                                    int max_state_items, int max_multi,
                                                    int max_slots, int s0_copy,
                                                    PlanHeader *__restrict__ hdr,
                                                    WorkItem *__restrict__ items,
                                                    WorkItem *__restrict__ sitems,
                                                    MultiSeq *__restrict__ multi) {
  extern __shared__ int smem[];
  const int nb = L / C + 1;  // chunk-count keys 0 .. L/C
  int *hist = smem;
  int *off = smem + nb;
  int *cursor = smem + 2 * nb;
  int *scratch = smem + 3 * nb;
  int *totals = smem + 3 * nb + 20;  // items, state items, split sequences, slots
  const int tid = threadIdx.x;

  for (int i = tid; i < nb; i += 1024) {
    hist[i] = 0;
    cursor[i] = 0;
  }
  if (tid < 4) totals[tid] = 0;
  __syncthreads();

  // Offsets are clamped to [0, T] so that malformed cu_seqlens can never send
  // a kernel outside the token arrays (the results are then meaningless).
  auto seq_start = [&](int n) -> int { return cu ? min(max(cu[n], 0), T) : n * T; };
  auto seq_len = [&](int n) -> int {
    if (!cu) return T;
    const int a = min(max(cu[n], 0), T);
    const int b = min(max(cu[n + 1], 0), T);
    return max(b - a, 0);
  };

  // 1. histogram of item chunk counts, and the totals
  for (int n = tid; n < N; n += 1024) {
    const int len = seq_len(n);
    const int nseg = max(1, (len + L - 1) / L);
    if (nseg > 1) atomicAdd(&hist[L / C], nseg - 1);
    const int last = len - (nseg - 1) * L;
    atomicAdd(&hist[(last + C - 1) / C], 1);
    atomicAdd(&totals[0], nseg);
    if (nseg > 1) {
      atomicAdd(&totals[1], (nseg - 1) * n_sub);
      atomicAdd(&totals[2], 1);
      atomicAdd(&totals[3], (nseg - 1) * n_sub + 1);
    }
  }
  __syncthreads();
  // Overlapping sequences (cu_seqlens not non-decreasing) can exceed the
  // capacities sized from T: then plan nothing rather than write out of range.
  if (totals[0] > max_items || totals[1] > max_state_items || totals[2] > max_multi ||
      totals[3] > max_slots) {
    if (tid == 0) {
      hdr->n_items = 0;
      hdr->n_state_items = 0;
      hdr->n_multi = 0;
    }
    return;
  }

  // 2. bucket offsets, longest items first: an exclusive scan of the
  // histogram from the highest key down, 1024 keys at a time
  int run = 0;
  for (int r0 = 0; r0 < nb; r0 += 1024) {
    const int r = r0 + tid, key = nb - 1 - r;
    int tot;
    const int ex = block_exclusive_scan_1024(r < nb ? hist[key] : 0, scratch, tot);
    if (r < nb) off[key] = run + ex;
    run += tot;
  }
  if (tid == 0) hdr->n_items = run;
  __syncthreads();

  // 3. emit items, 1024 sequences at a time
  int carry_slot = 0, carry_sitem = 0, carry_multi = 0;
  for (int base = 0; base < N; base += 1024) {
    const int n = base + tid;
    const bool valid = n < N;
    const int len = valid ? seq_len(n) : 0;
    const int nseg = valid ? max(1, (len + L - 1) / L) : 0;
    const bool split = nseg > 1;
    int ts, tsi, tm;
    const int e_slot = block_exclusive_scan_1024(split ? (nseg - 1) * n_sub + 1 : 0, scratch, ts);
    const int e_sitem = block_exclusive_scan_1024(split ? (nseg - 1) * n_sub : 0, scratch, tsi);
    const int e_multi = block_exclusive_scan_1024(split ? 1 : 0, scratch, tm);
    if (valid) {
      const int start = seq_start(n);
      const int slot_base = carry_slot + e_slot;
      for (int s = 0; s < nseg; ++s) {
        const int tb = start + s * L;
        const int te = min(tb + L, start + len);
        const int key = (te - tb + C - 1) / C;
        const int pos = off[key] + atomicAdd(&cursor[key], 1);
        WorkItem it;
        it.tok_begin = tb;
        it.tok_end = te;
        it.seq = n;
        // segment 0 reads S0 itself, or its copy in the chain's first slot
        // when S_T is S0 (the last segment, another workgroup, overwrites it)
        it.state_in = split && (s > 0 || s0_copy) ? slot_base + s * n_sub : -1;
        it.state_out = (s == nseg - 1) ? -1 : kNoStateOut;
        it.seq_begin = start;
        it.seq_end = start + len;
        it.pad = 0;
        items[pos] = it;
        if (split && s < nseg - 1) {  // non-last segments are full: L tokens
          for (int j = 0; j < n_sub; ++j) {
            WorkItem si = it;
            si.tok_begin = tb + j * Ls;
            si.tok_end = min(tb + (j + 1) * Ls, te);
            si.state_in = -1;
            si.state_out = slot_base + s * n_sub + j + 1;
            sitems[carry_sitem + e_sitem + s * n_sub + j] = si;
          }
        }
      }
      if (split) {
        MultiSeq m;
        m.seq = n;
        m.slot_base = slot_base;
        m.nslot = (nseg - 1) * n_sub + 1;
        m.pad = 0;
        multi[carry_multi + e_multi] = m;
      }
    }
    carry_slot += ts;
    carry_sitem += tsi;
    carry_multi += tm;
  }
  if (tid == 0) {
    hdr->n_state_items = carry_sitem;
    hdr->n_multi = carry_multi;
  }
}

// The same plan for a dense batch (no cu_seqlens) with at least two segments
// per sequence: every sequence has T tokens, so every sequence has the same
// segments and the plan is a closed form, written by one thread per
// (sequence, segment) without the histogram and scans. Full segments come
// first (longest first, as the counting sort orders them), then the last
// segments; slots, state items and split sequences in sequence order, as in
// plan_kernel.
__global__ __launch_bounds__(256) void plan_dense_kernel(int N, int T, int L, int Ls, int n_sub,
                                                         int s0_copy,
                                                         PlanHeader *__restrict__ hdr,
                                                         WorkItem *__restrict__ items,
                                                         WorkItem *__restrict__ sitems,
                                                         MultiSeq *__restrict__ multi) {
  const int nseg = (T + L - 1) / L;  // >= 2 where the host plans
  if (nseg < 2) {  // nothing to split: an empty plan
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      hdr->n_items = 0;
      hdr->n_state_items = 0;
      hdr->n_multi = 0;
    }
    return;
  }
  const int per_seq_slots = (nseg - 1) * n_sub + 1;
  const long total = (long)N * nseg;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    hdr->n_items = (int)total;
    hdr->n_state_items = N * (nseg - 1) * n_sub;
    hdr->n_multi = N;
  }
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    const int n = (int)(i / nseg), s = (int)(i % nseg);
    const int start = n * T;
    const int slot_base = n * per_seq_slots;
    const int tb = start + s * L;
    const int te = min(tb + L, start + T);
    WorkItem it;
    it.tok_begin = tb;
    it.tok_end = te;
    it.seq = n;
    it.state_in = (s > 0 || s0_copy) ? slot_base + s * n_sub : -1;
    it.state_out = (s == nseg - 1) ? -1 : kNoStateOut;
    it.seq_begin = start;
    it.seq_end = start + T;
    it.pad = 0;
    items[s < nseg - 1 ? n * (nseg - 1) + s : N * (nseg - 1) + n] = it;
    if (s < nseg - 1) {
      for (int j = 0; j < n_sub; ++j) {
        WorkItem si = it;
        si.tok_begin = tb + j * Ls;
        si.tok_end = min(tb + (j + 1) * Ls, te);
        si.state_in = -1;
        si.state_out = slot_base + s * n_sub + j + 1;
        sitems[(n * (nseg - 1) + s) * n_sub + j] = si;
      }
    }
    if (s == 0) {
      MultiSeq m;
      m.seq = n;
      m.slot_base = slot_base;
      m.nslot = per_seq_slots;
      m.pad = 0;
      multi[n] = m;
    }
  }
}

// Chain the state pieces: from S0 (or 0) as the state before piece 0, for b >= 1
//   slot[base+b] = exp(gamma[base+b]) * slot[base+b-1] + slot[base+b]
// where the state pass left piece b-1's local state and total log-decay in
// slot base+b. Only the starts of segments after the first (b a positive
// multiple of n_sub) are read afterwards, so only they are written back; the
// first segment starts from S0 itself, or (s0_copy, when the output pass
// writes S_T over S0) from a copy of it in slot base. One thread per four
// consecutive state elements.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ S0,
                                                      const PlanHeader *__restrict__ hdr,
                                                      const MultiSeq *__restrict__ multi,
                                                      float *__restrict__ slots,
                                                      const float *__restrict__ slot_gamma,
                                                      int H, int dkdv, int n_sub, int s0_copy) {
  const int bph = dkdv / 1024;  // blocks per (sequence, head)
  const int m = blockIdx.x / (H * bph);
  if (m >= hdr->n_multi) return;
  const int h = (blockIdx.x / bph) % H;
  const int e = (blockIdx.x % bph) * 1024 + threadIdx.x * 4;
  const MultiSeq ms = multi[m];
  f32x4 cur = {0.f, 0.f, 0.f, 0.f};
  if (S0) cur = *reinterpret_cast<const f32x4 *>(S0 + ((size_t)ms.seq * H + h) * dkdv + e);
  if (s0_copy)
    *reinterpret_cast<f32x4 *>(slots + ((size_t)ms.slot_base * H + h) * dkdv + e) = cur;
  // eight pieces at a time: their loads all issued before the chain's stores
  // (which the compiler would otherwise wait for before each next load);
  // indexes past the last piece are clamped to it and their values unused
  for (int s0 = 1; s0 < ms.nslot; s0 += 8) {
    f32x4 val[8];
    float lgam[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sl = ms.slot_base + min(s0 + j, ms.nslot - 1);
      val[j] = *reinterpret_cast<const f32x4 *>(slots + ((size_t)sl * H + h) * dkdv + e);
      lgam[j] = slot_gamma[(size_t)sl * H + h];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j < ms.nslot) {
        const int sl = ms.slot_base + s0 + j;
        cur = expf(lgam[j]) * cur + val[j];
        if ((s0 + j) % n_sub == 0)
          *reinterpret_cast<f32x4 *>(slots + ((size_t)sl * H + h) * dkdv + e) = cur;
      }
    }
  }
}

hipError_t launch_plan(const int32_t *cu_seqlens, const FwdDims &d, const PlanLayout &lay,
                       bool s0_copy, void *workspace, hipStream_t stream) {
  char *ws = static_cast<char *>(workspace);
  if (!cu_seqlens) {  // dense: the closed-form plan (make_plan plans only split batches)
    const long total = (long)d.N * ((d.T + lay.seg_len - 1) / lay.seg_len);
    // at least one block: it writes the header (an empty plan has no items)
    const int blocks = (int)std::max<long>(1, std::min<long>((total + 255) / 256, 1024));
    hipLaunchKernelGGL(plan_dense_kernel, dim3(blocks), dim3(256), 0, stream, d.N, d.T,
                       lay.seg_len, lay.sub_len, lay.n_sub, (int)s0_copy,
                       reinterpret_cast<PlanHeader *>(ws + lay.off_header),
                       reinterpret_cast<WorkItem *>(ws + lay.off_items),
                       reinterpret_cast<WorkItem *>(ws + lay.off_state_items),
                       reinterpret_cast<MultiSeq *>(ws + lay.off_multi));
    return hipGetLastError();
  }
  const int nb = lay.seg_len / d.C + 1;
  const size_t lds = sizeof(int) * (3 * nb + 32);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), lds, stream, cu_seqlens, d.N, d.T,
                     lay.seg_len, d.C, lay.sub_len, lay.n_sub, lay.max_items,
                     lay.max_state_items, lay.max_multi,
                     lay.max_slots, (int)s0_copy,
                     reinterpret_cast<PlanHeader *>(ws + lay.off_header),
                     reinterpret_cast<WorkItem *>(ws + lay.off_items),
                     reinterpret_cast<WorkItem *>(ws + lay.off_state_items),
                     reinterpret_cast<MultiSeq *>(ws + lay.off_multi));
  return hipGetLastError();
}

hipError_t launch_combine(const float *S0, const FwdDims &d, const PlanLayout &lay,
                          bool s0_copy, void *workspace, hipStream_t stream) {
  if (lay.max_multi == 0) return hipSuccess;
  char *ws = static_cast<char *>(workspace);
  const int dkdv = d.dk * d.dv;
  const long blocks = (long)lay.max_multi * d.H * (dkdv / 1024);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, stream, S0,
                     reinterpret_cast<const PlanHeader *>(ws + lay.off_header),
                     reinterpret_cast<const MultiSeq *>(ws + lay.off_multi),
                     reinterpret_cast<float *>(ws + lay.off_slots),
                     reinterpret_cast<const float *>(ws + lay.off_slot_gamma), d.H, dkdv,
                     lay.n_sub, (int)s0_copy);
  return hipGetLastError();
}

}  // namespace gla
