// Host-side work planning of the chunked forward: the work-item and workspace
// structures shared with the device planner, how long segments are, the
// workspace layout, and the argument helpers. Plain C++ (no HIP), so that it
// also builds into the host sanitizer test.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "gla.h"

namespace gla {

// One unit of chunked-forward work for one (head, dv-slice): a run of tokens
// [tok_begin, tok_end) of sequence `seq` on the flattened time axis (row b of
// a dense batch starts at b*T). `state_in` < 0 starts from S0[seq] (zeros if
// S0 is NULL); otherwise from workspace state slot `state_in`. In the
// output pass, `state_out` < 0 writes the final state to S_T[seq] and
// `state_out` == kNoStateOut writes nothing; in the state pass it is the slot
// that receives the segment's local state and total log-decay.
struct WorkItem {
  int tok_begin;
  int tok_end;
  int seq;
  int state_in;
  int state_out;
  int seq_begin, seq_end;  // the whole sequence's tokens (time-reversed runs map through them)
  int pad;
};
constexpr int kNoStateOut = -2;

// A sequence split into segments: its chain of `nslot` state slots starts at
// slot_base (slot_base holds S0; slot_base + b the state after b state items,
// each a sub-segment of sub_len tokens of a non-last segment; segment s starts
// from slot_base + s * (sub-segments per segment)).
struct MultiSeq {
  int seq;
  int slot_base;
  int nslot;
  int pad;
};

struct PlanHeader {
  int n_items;        // output-pass items
  int n_state_items;  // state-pass items (all non-last segments)
  int n_multi;        // sequences with more than one segment
  int pad;
};

// Workspace layout of a planned forward (all offsets 256-byte aligned).
struct PlanLayout {
  int seg_len;          // tokens per segment (multiple of the chunk size)
  int sub_len;          // tokens per state-pass item (divides the segment into n_sub pieces)
  int n_sub;            // state-pass items per non-last segment
  int max_items;        // bound on output-pass items
  int max_state_items;  // bound on state-pass items
  int max_multi;        // bound on split sequences
  int max_slots;        // bound on state slots
  size_t off_header, off_items, off_state_items, off_multi, off_slots, off_slot_gamma;
  size_t total_bytes;
};

// The planning functions take the device's CU count (n_cu) as an argument.
inline bool supported_head_dim(int d) { return d == 64 || d == 128; }

// (d_k, d_v) pairs of the forward and decode: any of {64, 128} x {64, 128},
// and Laplace 3B's 96 x 192 heads.
inline bool fwd_dims(int dk, int dv) {
  return (supported_head_dim(dk) && supported_head_dim(dv)) || (dk == 96 && dv == 192);
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int round_up(long x, int m) { return (int)(((x + m - 1) / m) * m); }

// Chunk sizes of the chunked form the calls accept (Laplace 3B on AWS
// Trainium2: 128-token chunks in "Challenge 1", 256 discussed in "Challenge 3").
inline bool supported_chunk(int c) { return c == 64 || c == 128 || c == 256; }

// The chunk the kernels run at. A chunk of C tokens of the chunked form equals
// C / C' consecutive chunks of C' tokens in exact arithmetic (the state
// advance composes). The bf16 matrix-core kernel tiles 64 tokens, whose Q, K,
// V tiles double-buffer in LDS (at 128 they do not), so it runs every chunk
// size as 64-token chunks; the fp32 kernel runs 64 and 128 as asked and 256 as
// two chunks of 128.
inline int kernel_chunk(gla_dtype in_dtype, bool f32_kernel, int chunk_size) {
  if (in_dtype == GLA_BF16 && !f32_kernel) return 64;
  return chunk_size > 128 ? 128 : chunk_size;  // a 256-token chunk is two of 128
}

// State columns one workgroup of the forward owns (the column "slice"): 96 for
// the twelve-wavefront bf16 kernel (d_k = 96, chunk 64), else 64 (bf16) or 32.
inline int slice_width(gla_dtype in_dtype, int dk, int C) {
  if (in_dtype != GLA_BF16) return 32;
  return dk == 96 && C == 64 ? 96 : 64;
}

// Tokens per work item. A dense batch with enough (sequence, head, slice)
// work units to cover every CU runs each sequence whole; otherwise sequences
// are split into about ceil(CUs / units) segments. A packed batch caps
// segments at its per-CU share of the work, so no single long sequence sets
// the critical path. GLA_SEG_LEN overrides the choice (tuning only; the
// result does not depend on it beyond rounding).
inline int choose_seg_len(int B, int T, int H, int dk, int dv, int N, int C, bool has_cu,
                          int n_cu, gla_dtype in_dtype) {
  long L;
  const char *env = std::getenv("GLA_SEG_LEN");
  const int n_slices = dv / slice_width(in_dtype, dk, C);
  if (env && std::atoi(env) > 0) {
    L = std::atoi(env);
  } else if (!has_cu) {
    const long units = (long)B * H * n_slices;
    // workgroups to aim for: one per CU on the bf16 kernels, four on the
    // fp32 one (two fit per CU, and it is bound by latency, not bandwidth),
    // except with 192-dim keys (the 96 x 192 backward's dq and dk runs), whose
    // chunks carry enough work that a split costs more than it hides
    // (laplace_2k backward: 3.82 ms whole against 4.04 ms in three segments)
    const long target = (long)n_cu * (in_dtype == GLA_BF16 || dk == 192 ? 1 : 4);
    if (units >= target) {
      L = T;
    } else {
      const long nseg = (target + units - 1) / units;
      L = (T + nseg - 1) / nseg;
    }
    if (in_dtype == GLA_BF16) {
      // A split adds three launches (plan, state pass, combine) and a combine
      // chain that is sequential in the segments of a sequence, so on the
      // matrix-core kernels short segments do not pay: a sequence of at most
      // 8 chunks (chunk 64) or 2 (chunk 128) runs whole, and at chunk 64
      // segments keep about sqrt(chunks) / 1.7 chunks (measured on MI355X for
      // 256 - 4,096 tokens and 1 - 64 work units; the fp32 kernel, several
      // times slower per chunk, always gains from the split).
      const long chunks = ((long)T + C - 1) / C;
      if (chunks <= (C == 64 ? 8 : 2)) {
        L = T;
      } else if (C == 64) {
        const long seg_chunks = std::max(1L, std::lround(std::sqrt((double)chunks) / 1.7));
        L = std::max(L, seg_chunks * C);
      }
    }
  } else {
    // the dense rule's per-CU target, 192-dim keys included
    const long work = (long)T * H * n_slices;
    L = work / ((long)n_cu * (in_dtype == GLA_BF16 || dk == 192 ? 1 : 4));
    if (in_dtype == GLA_BF16 && C == 64 && N > 0) {
      // the segment floor of dense batches, from the mean sequence length
      // (the lengths themselves stay on the device)
      const double mean_chunks = (double)T / N / C;
      const long seg_chunks = std::max(1L, std::lround(std::sqrt(mean_chunks) / 1.7));
      L = std::max(L, seg_chunks * C);
    }
  }
  // clamp in long before rounding (the per-CU share of a huge packed batch
  // exceeds int): C <= L <= min(T rounded up, 65536), then a multiple of C
  // (65536 bounds the scheduler's sort buckets; a multiple of both chunk sizes)
  const long cap = (((long)std::max(T, C) + C - 1) / C) * C;
  L = std::min(std::max(L, (long)C), std::min(cap, 65536L));
  return (int)(((L + C - 1) / C) * C);
}

// Whether the forward needs the device-side planner, and its workspace layout.
inline bool make_plan(int B, int T, int H, int dk, int dv, int N, int C, bool has_cu,
                      int n_cu, gla_dtype in_dtype, PlanLayout &lay) {
  std::memset(&lay, 0, sizeof(lay));
  const int L = choose_seg_len(B, T, H, dk, dv, N, C, has_cu, n_cu, in_dtype);
  lay.seg_len = L;
  long seg_items;  // (a bound on) the non-last segments, each one state-pass run
  if (!has_cu) {
    const int nseg = T > 0 ? (T + L - 1) / L : 1;
    if (nseg <= 1) return false;
    seg_items = (long)B * (nseg - 1);
  } else {
    seg_items = T / L;  // segments that can be full length
  }
  // The state pass runs each non-last segment in n_sub pieces so that it has
  // at least about four workgroups per CU (pieces of at least 8 chunks); the
  // combine then chains the pieces. GLA_STATE_SUB overrides n_sub (tuning and
  // tests; results do not depend on it beyond rounding).
  int want = 1;
  if (seg_items > 0) {
    const long units = seg_items * H * (dv / slice_width(in_dtype, dk, C));
    want = (int)((4L * n_cu + units - 1) / units);
    want = std::min(want, std::max(1, L / (8 * C)));
  }
  const char *env = std::getenv("GLA_STATE_SUB");
  if (env && std::atoi(env) > 0) want = std::atoi(env);
  want = std::max(1, std::min(want, L / C));
  lay.sub_len = round_up((L + want - 1) / want, C);
  lay.n_sub = (L + lay.sub_len - 1) / lay.sub_len;
  if (!has_cu) {
    lay.max_items = (int)(seg_items + B);
    lay.max_state_items = (int)(seg_items * lay.n_sub);
    lay.max_multi = B;
    lay.max_slots = (int)(seg_items * lay.n_sub + B);
  } else {
    lay.max_items = (int)(N + seg_items);
    lay.max_state_items = (int)(seg_items * lay.n_sub);
    lay.max_multi = (int)seg_items;
    lay.max_slots = (int)(seg_items * (lay.n_sub + 1));
  }
  size_t off = 0;
  lay.off_header = off;
  off = align256(off + sizeof(PlanHeader));
  lay.off_items = off;
  off = align256(off + sizeof(WorkItem) * (size_t)lay.max_items);
  lay.off_state_items = off;
  off = align256(off + sizeof(WorkItem) * (size_t)lay.max_state_items);
  lay.off_multi = off;
  off = align256(off + sizeof(MultiSeq) * (size_t)lay.max_multi);
  lay.off_slots = off;
  off = align256(off + sizeof(float) * (size_t)lay.max_slots * H * dk * dv);
  lay.off_slot_gamma = off;
  off = align256(off + sizeof(float) * (size_t)lay.max_slots * H);
  lay.total_bytes = off;
  return true;
}

inline bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}


}  // namespace gla
