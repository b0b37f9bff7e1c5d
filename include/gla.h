/*
 * gla.h - C ABI of libgla.so: gated linear attention (GLA) on AMD MI355X (gfx950).
 *
 * The method (Laplace 3B on AWS Trainium2, automationscribe.com/?p=7116,
 * section "GLA mixer"): every head keeps a d_k x d_v matrix state that decays
 * and absorbs the rank-1 outer product of the current key and value, and the
 * output reads the state with the query. With a per-token, per-head gate
 * g_t = exp(l_t):
 *
 *     S_t = g_t * S_{t-1} + k_t^T v_t          (S is d_k x d_v, row-major)
 *     o_t = q_t S_t                            (after the update)
 *
 * No 1/sqrt(d_k) scale and no normaliser are applied: callers fold any scale
 * into k (or q). The page's fixed per-head decay lambda_h is the special case
 * l_t = ln(lambda_h).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (HBM of the current device),
 *    dense and row-major in the layouts given, allocated and owned by the
 *    caller. The library allocates no device memory and keeps no state
 *    between calls; it is re-entrant, and calls on different streams do not
 *    interact. Calls on the same buffers from two streams race.
 *  - Alignment: every tensor and workspace pointer must be 16-byte aligned,
 *    except the fp32 log-gate streams (g, log_lambda, dlog_g) and the int32
 *    arrays (cu_seqlens, slots), which need 4-byte alignment. (Fresh
 *    allocations of HIP and of PyTorch's caching allocator are 256-byte
 *    aligned; a view with a storage offset may not be.) A misaligned pointer
 *    returns GLA_ERR_INVALID_ARGUMENT.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it and the call returns without synchronising.
 *  - Argument errors are detected on the host before anything is enqueued and
 *    reported by the return value; nothing is written then. A failed kernel
 *    launch returns GLA_ERR_HIP. Faults inside a kernel surface at the
 *    caller's next synchronisation, as with any HIP library.
 *  - Tensor values are not validated: NaN/Inf propagate, and l_t > 0 (a
 *    growing state) is computed as given.
 *  - Reset gates: l_t = -inf (g_t = 0) is allowed and resets the state,
 *    S_t = k_t^T v_t, exactly, in every entry point. Any l_t <= -128 ln 2
 *    (about -88.72, i.e. g_t <= 2^-128, below the smallest normal fp32) is
 *    treated the same way: g_t = 0 exactly. No decay product that spans a
 *    reset is formed, so a reset never turns into NaN; the backward returns
 *    dlog_g = 0 at a reset and no gradient crosses it.
 *  - Supported sizes: d_k, d_v in {64, 128}; chunk_size in {64, 128, 256}. The
 *    forward, the backward and the decode steps also take (d_k, d_v) =
 *    (96, 192), the head shape of Laplace 3B ("GLA mixer"). Anything else
 *    returns GLA_ERR_UNSUPPORTED.
 */
#ifndef GLA_H_
#define GLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GLA_OK = 0,
  GLA_ERR_INVALID_ARGUMENT = 1, /* null or misaligned pointer, negative size, bad dtype,
                                   o aliasing an input */
  GLA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (head dims, chunk size) */
  GLA_ERR_WORKSPACE = 3,        /* workspace NULL or smaller than the size query returns */
  GLA_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} gla_status;

typedef enum {
  GLA_F32 = 0, /* IEEE binary32 */
  GLA_BF16 = 1 /* bfloat16 (upper half of binary32), round-to-nearest-even on output */
} gla_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char *gla_status_string(gla_status s);

/*
 * Chunked-parallel forward (prefill / training forward) over a dense or
 * packed batch. Computes the recurrence above in its chunked form (Laplace 3B
 * on AWS Trainium2, "Challenge 1": within each chunk of `chunk_size` tokens
 * the output is decay-masked linear attention plus the query read of the
 * running state; the state then advances by the decay compounded over the
 * chunk). Chunks restart at every sequence start; the last chunk of a
 * sequence may be partial.
 *
 *   q          [B, T, H, dk]  in_dtype
 *   k          [B, T, H, dk]  in_dtype
 *   v          [B, T, H, dv]  in_dtype
 *   g          [B, T, H]      fp32 natural-log gates l_t (the gate is exp(l_t))
 *   S0         [N, H, dk, dv] fp32 initial states, or NULL for zeros
 *   cu_seqlens [N+1] int32 DEVICE array of sequence offsets into the time axis,
 *              or NULL. With cu_seqlens, B must be 1, cu_seqlens[0] = 0,
 *              offsets non-decreasing and cu_seqlens[N] = T (these values are
 *              read on the device and are not checked). Without it, N = B and
 *              every row of the batch is one sequence of length T.
 *   o          [B, T, H, dv]  out_dtype (GLA_F32 carries full accuracy; GLA_BF16
 *              rounds the fp32 result once). Must not overlap any input.
 *   S_T        [N, H, dk, dv] fp32 final states, or NULL to skip. May be the
 *              same pointer as S0 (each state is read before it is written);
 *              any other overlap with an input is undefined.
 *   num_seqs   N (must equal B when cu_seqlens is NULL).
 *   chunk_size 64, 128 or 256: the chunk length C of the chunked form
 *              ("Challenge 1" chunks by 128 tokens; "Challenge 3" weighs
 *              256). Results agree across chunk sizes up to rounding: a chunk
 *              of C tokens equals consecutive shorter chunks in exact
 *              arithmetic, and the kernels run bf16 inputs as 64-token chunks
 *              and fp32 inputs as chunks of min(C, 128) tokens.
 *   in_dtype   GLA_BF16 (MFMA path, fp32 accumulation and fp32 state) or
 *              GLA_F32 (fp32 arithmetic throughout).
 *   workspace  device scratch of at least gla_fwd_chunked_workspace_size()
 *              bytes (may be NULL when that size is 0); contents on entry do
 *              not matter; it is in use until the enqueued work completes.
 */
size_t gla_fwd_chunked_workspace_size(int B, int T, int H, int dk, int dv, int num_seqs,
                                      int chunk_size, int has_cu_seqlens, gla_dtype in_dtype);

gla_status gla_fwd_chunked(const void *q, const void *k, const void *v, const float *g,
                           const float *S0, const int32_t *cu_seqlens, void *o, float *S_T,
                           int B, int T, int H, int dk, int dv, int num_seqs, int chunk_size,
                           gla_dtype in_dtype, gla_dtype out_dtype, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * gla_fwd_chunked without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Same arguments, results, checks and errors as
 * gla_fwd_chunked, minus workspace / workspace_bytes: the scratch the call
 * needs (gla_fwd_chunked_workspace_size for the same sizes; 0 for dense
 * batches that fill the GPU) comes from a fixed array of
 * gla_fwd_chunked_noalloc_max_scratch() bytes (64 MiB) that the library holds
 * on each GPU it runs on until the process ends. A call that needs more
 * returns GLA_ERR_WORKSPACE before anything is enqueued (use
 * gla_fwd_chunked with a workspace then). The call allocates nothing (no
 * hipMalloc, no library allocation); its first call on a device looks up
 * that device's address of the array. Every call on one GPU shares the
 * array: calls that may overlap in time on one GPU (other streams, other
 * host threads) race and must be ordered by the caller. Nothing in it needs
 * to start zeroed; its contents after a call are undefined.
 */
size_t gla_fwd_chunked_noalloc_max_scratch(void);

gla_status gla_fwd_chunked_noalloc(const void *q, const void *k, const void *v, const float *g,
                                   const float *S0, const int32_t *cu_seqlens, void *o,
                                   float *S_T, int B, int T, int H, int dk, int dv,
                                   int num_seqs, int chunk_size, gla_dtype in_dtype,
                                   gla_dtype out_dtype, void *stream);

/*
 * The same forward for fixed per-head decays (Laplace 3B on AWS Trainium2,
 * "Decay schedule": each head's decay is set at initialisation on a
 * geometric schedule and not learned), so there is no per-token gate stream:
 * every token of head h has l_t = log_lambda[h].
 *
 *   log_lambda [H] fp32 device array of natural-log decays ln(lambda_h).
 *
 * Every other argument, the workspace (gla_fwd_chunked_workspace_size with
 * the same sizes), the supported sizes and the errors are as in
 * gla_fwd_chunked; results equal gla_fwd_chunked with g[b, t, h] =
 * log_lambda[h] up to rounding.
 */
gla_status gla_fwd_chunked_fixed_decay(const void *q, const void *k, const void *v,
                                       const float *log_lambda, const float *S0,
                                       const int32_t *cu_seqlens, void *o, float *S_T, int B,
                                       int T, int H, int dk, int dv, int num_seqs,
                                       int chunk_size, gla_dtype in_dtype, gla_dtype out_dtype,
                                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward of gla_fwd_chunked (training; Laplace 3B on AWS Trainium2,
 * "Challenge 3: Backward-pass unrolling for a sequential recurrence": the
 * training step differentiates through the chunk-by-chunk state updates). For upstream gradients dO of o and dS_T of S_T it returns
 * the gradients of L = sum <dO, o> + sum <dS_T, S_T>:
 *
 *   dq, dk [B, T, H, dk] fp32;  dv [B, T, H, dv] fp32
 *   dg     [B, T, H]     fp32   gradient with respect to the log-gates l_t
 *   dS0    [N, H, dk, dv] fp32  gradient with respect to S0, or NULL to skip
 *
 * Inputs q, k, v, g, S0, cu_seqlens, B, T, H, dk, dv, num_seqs, chunk_size
 * and in_dtype exactly as for the forward (the forward's results are not
 * needed; the states are recomputed). dO [B, T, H, dv] is in_dtype; dS_T
 * [N, H, dk, dv] fp32, or NULL for zero. Method: dq is a forward run on the
 * transposed state; dk and dv are forward runs over each sequence reversed
 * in time (the adjoint dL/dS_t obeys the same recurrence backwards, with the
 * gates shifted by one token); dg follows from dL/dB_t = q_t.dq_t - k_t.dk_t
 * (B the cumulative log-gate, plus <dS_T, S_T> at a sequence's last token)
 * summed over later tokens of the sequence. Head shapes: (dk, dv) in
 * {64, 128} x {64, 128}, and 96 x 192 (Laplace 3B's heads; its dq and dk runs
 * have 192-dim keys and run on the fp32-arithmetic kernel, which reads bf16
 * inputs as they are); others give GLA_ERR_UNSUPPORTED.
 * Outputs must not overlap the inputs or each other. The workspace
 * (gla_bwd_chunked_workspace_size bytes, never 0 for a non-empty batch) holds
 * transposed states, the adjoint after the first token, per-token partial
 * sums and the forward runs' plans; its contents on entry do not matter.
 * Errors as gla_fwd_chunked.
 */
size_t gla_bwd_chunked_workspace_size(int B, int T, int H, int dk, int dv, int num_seqs,
                                      int chunk_size, int has_cu_seqlens, gla_dtype in_dtype);

gla_status gla_bwd_chunked(const void *q, const void *k, const void *v, const float *g,
                           const float *S0, const int32_t *cu_seqlens, const void *dO,
                           const float *dS_T, float *dq, float *dk, float *dv, float *dg,
                           float *dS0, int B, int T, int H, int dk_dim, int dv_dim, int num_seqs,
                           int chunk_size, gla_dtype in_dtype, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * One recurrent decode step for N independent sequences (Laplace 3B on AWS
 * Trainium2, "GLA mixer" for the update and readout; "Inference optimization"
 * for serving with one fixed-size state per sequence):
 *
 *   S[n,h] <- exp(g[n,h]) * S[n,h] + k[n,h]^T v[n,h]      (in place)
 *   o[n,h]  = q[n,h] S[n,h]                              (updated state)
 *
 *   q [N, H, dk], k [N, H, dk], v [N, H, dv]   in_dtype (GLA_BF16 or GLA_F32)
 *   g [N, H]           fp32 natural-log gates; -inf gives g = 0 (a reset)
 *   S [N, H, dk, dv]   fp32 states, read and overwritten in place
 *   o [N, H, dv]       out_dtype; must not overlap S or the inputs
 */
gla_status gla_decode_step(const void *q, const void *k, const void *v, const float *g,
                           float *S, void *o, int N, int H, int dk, int dv, gla_dtype in_dtype,
                           gla_dtype out_dtype, void *stream);

/*
 * The decode step over a serving pool of states (Laplace 3B on AWS Trainium2,
 * "Inference optimization": the serving engine keeps one fixed-size state per
 * sequence in its pool and decodes fixed-width, padded batches). Request n
 * uses pool entry slots[n]:
 *
 *   S_pool[slots[n], h] <- exp(g[n,h]) * S_pool[slots[n], h] + k[n,h]^T v[n,h]
 *   o[n, h]              = q[n,h] S_pool[slots[n], h]          (updated state)
 *
 *   S_pool [P, H, dk, dv] fp32, updated in place at the requested slots only
 *   slots  [N] int32 DEVICE array; a slot outside [0, P) (e.g. -1) marks a
 *          padded lane: no state is read or written and o[n] is set to 0.
 *          Valid slots must be distinct (two requests on one slot race).
 *   order  [2, N] int32 DEVICE array or NULL: the order in which the
 *          requests' states are streamed, as gla_decode_slot_order writes it
 *          for these slots (row 0 the requests, row 1 their slots, which the
 *          step then reads in place of slots[]). The results do not depend
 *          on it; the time does: states streamed in that order run near the
 *          dense step's rate, states in a random slot order about 6% slower.
 *          Entries of row 0 outside [0, N) are skipped; anything but a
 *          permutation of 0 .. N-1 there leaves outputs unwritten or updates
 *          a state twice.
 *   q, k, v, g, o, N, H, dk, dv, dtypes as gla_decode_step.
 */
gla_status gla_decode_step_slots(const void *q, const void *k, const void *v, const float *g,
                                 float *S_pool, const int32_t *slots, const int32_t *order,
                                 void *o, int N, int P, int H, int dk, int dv, gla_dtype in_dtype,
                                 gla_dtype out_dtype, void *stream);

/*
 * The streaming order for a serving batch (Laplace 3B on AWS Trainium2,
 * "Inference optimization": the engine decodes a batch of sequences whose
 * states sit in fixed pool slots): order[0][0 .. N-1] = the requests 0 .. N-1
 * sorted by the pool position of their slot, padded lanes (slots outside
 * [0, P)) last, and order[1][i] = slots[order[0][i]]. slot_bytes is the size
 * of one pool entry (H * dk * dv * 4). Where it divides 4 MiB and the pool
 * holds at least three whole 4 MiB blocks of entries, the pool is streamed
 * the way the dense decode step streams a batch: block by block, consecutive
 * blocks in the order s apart (block b at rank b * s^-1 mod the block count,
 * s the first of 3, 5, 7, ... coprime with it), slot order within a block,
 * and the entries past the last whole block after all blocks; otherwise
 * (slot_bytes 0, other sizes, small pools) plain ascending slot order. Every
 * layer of a step uses the same slots, so one call per step serves all of
 * them. One workgroup; device arrays slots [N] and order [2, N] (must not
 * overlap). P <= 32768, else GLA_ERR_UNSUPPORTED (pass order = NULL to the
 * decode calls instead). Requests sharing a slot are ordered arbitrarily.
 */
gla_status gla_decode_slot_order(const int32_t *slots, int N, int P, size_t slot_bytes,
                                 int32_t *order, void *stream);

/*
 * Token-mixer epilogue around the readout (Laplace 3B on AWS Trainium2,
 * "GLA mixer"), in one pass: per token t and head h,
 *
 *   o'  = o + sigmoid(sum_i q_i a[h,i] k_i) v          (self-augmentation;
 *                                                        a = 0 adds v / 2)
 *   z   = o' / sqrt(mean_j o'_j^2 + eps) * rms_w[h] * silu(g),
 *   silu(x) = x * sigmoid(x)
 *
 * i.e. the head's RMSNorm over its d_v outputs (the heads of one decay tier
 * pass the same weight row) and the SiLU output gate. The output projection
 * that follows on the page is not part of this call.
 *
 *   o        [n_tokens, H, dv]  o_dtype (the forward's or decode's output)
 *   q, k     [n_tokens, H, dk]  in_dtype
 *   v, g     [n_tokens, H, dv]  in_dtype (g: the head's slice of the gate stream)
 *   a        [H, dk]  fp32 self-augmentation scales
 *   rms_w    [H, dv]  fp32 RMSNorm weights per head
 *   eps      finite, >= 0
 *   z        [n_tokens, H, dv]  out_dtype; may be o itself when out_dtype ==
 *            o_dtype (in place), must not overlap anything else.
 *
 * Sizes: (dk, dv) as the forward. n_tokens = B * T for a [B, T, H, d] batch,
 * or N for one decode step.
 */
gla_status gla_mixer_epilogue(const void *o, const void *q, const void *k, const void *v,
                              const void *g, const float *a, const float *rms_w, float eps,
                              void *z, int n_tokens, int H, int dk, int dv, gla_dtype o_dtype,
                              gla_dtype in_dtype, gla_dtype out_dtype, void *stream);

/*
 * One decode step with the token-mixer epilogue fused (Laplace 3B on AWS
 * Trainium2, "GLA mixer" and "Inference optimization"): the state update of
 * gla_decode_step (slots == NULL: S is [N, H, dk, dv]) or of
 * gla_decode_step_slots (slots != NULL: S is the pool [P, H, dk, dv]; order
 * as there, NULL without slots), then
 * gla_mixer_epilogue's arithmetic on the readout, in one kernel; the readout
 * o itself is not written.
 *
 *   q, k [N, H, dk], v [N, H, dv], g [N, H] fp32: as gla_decode_step
 *   g_out [N, H, dv] in_dtype   the gate stream of the epilogue
 *   a [H, dk], rms_w [H, dv]    fp32, eps finite >= 0: as gla_mixer_epilogue
 *   z [N, H, dv] out_dtype      the epilogue's output (padded lanes: 0)
 *
 * Sizes and dtypes as gla_decode_step. z must not overlap anything; S must not
 * overlap the inputs.
 */
gla_status gla_decode_mixer(const void *q, const void *k, const void *v, const float *g,
                            float *S, const int32_t *slots, const int32_t *order, int P,
                            const void *g_out,
                            const float *a, const float *rms_w, float eps, void *z, int N, int H,
                            int dk, int dv, gla_dtype in_dtype, gla_dtype out_dtype,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H_ */
