"""fp64 CPU oracle for the gated linear-attention (GLA) recurrence.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module: only the tests, the package's smoke check and the benchmark's
CPU-baseline leg do. It shares no code with the HIP path; the two meet only
in the seeded input generator.

What it computes is the plain definition, one token at a time, in fp64:

    S_t = g_t * S_{t-1} + k_t^T v_t,      o_t = q_t S_t,      g_t = exp(l_t)

per (sequence, head), with S a d_k x d_v matrix (row-major, o a row vector).
Source: Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), section
"GLA mixer": each head keeps a d_k x d_v matrix state that is decayed and
then receives the rank-1 outer product of the current key and value; the
readout queries that state with q_t. The page's equation images are lost;
its fixed per-head decay is generalised to a per-token, per-head scalar gate
(the fixed decay is the special case l_t = ln(lambda_h)). Readings taken
where the page is silent:
  * the readout is inclusive: o_t reads S_t, after token t's update;
  * the gate multiplies the old state only, not the current k_t^T v_t;
  * the gate is passed as its natural log l_t (fp32); l_t = -inf is a reset;
  * no 1/sqrt(d_k) scale and no normaliser inside the method;
  * packed (varlen) batches restart the state at every sequence start,
    from that sequence's own S0 (zeros when S0 is None).

All inputs are converted exactly to fp64 (bf16 and fp32 values embed in
fp64 without rounding). Pins: tests/test_oracle_pins.py (brute-force masked
sum, no-decay and fixed-decay closed forms, exact rationals, reset,
continuation, linearity, chunked regrouping) and tests/test_oracle_mutants.py.

The backward (recurrent_backward) is the reverse-mode adjoint of the same
token-by-token recurrence, written out: it walks each sequence backwards
carrying dL/dS_t. Its pins (tests/test_oracle_bwd_pins.py) are central finite
differences and fp64 automatic differentiation of an independent forward.
"""
from __future__ import annotations

import numpy as np

__all__ = ["recurrent_forward", "recurrent_backward", "decode_step", "normwise_error"]


def _seq_bounds(B: int, T: int, cu_seqlens):
    """(row, start, end) for every sequence of a dense or packed batch."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if B != 1:
        raise ValueError("a packed batch has B == 1")
    return [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


def recurrent_forward(q, k, v, log_g, S0=None, cu_seqlens=None, heads=None):
    """Token-by-token GLA forward in fp64.

    q, k: [B, T, H, dk]; v: [B, T, H, dv]; log_g: [B, T, H] natural-log gates;
    S0: [N, H, dk, dv] or None (zeros); cu_seqlens: [N+1] offsets into the
    packed time axis (then B == 1) or None (N = B sequences of length T).
    heads: optional list of head indices to evaluate (heads are independent);
    the outputs then carry only those heads, in that order.

    Returns (o [B, T, H', dv] fp64, S_T [N, H', dk, dv] fp64).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    log_g = np.asarray(log_g)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    hs = np.arange(H) if heads is None else np.asarray(heads, dtype=np.int64)
    bounds = _seq_bounds(B, T, cu_seqlens)
    o = np.zeros((B, T, len(hs), dv), dtype=np.float64)
    S_T = np.zeros((len(bounds), len(hs), dk, dv), dtype=np.float64)
    for n, (b, start, end) in enumerate(bounds):
        if S0 is None:
            S = np.zeros((len(hs), dk, dv), dtype=np.float64)
        else:
            S = np.asarray(S0)[n][hs].astype(np.float64)
        for t in range(start, end):
            g = np.exp(log_g[b, t, hs].astype(np.float64))           # [H']
            kt = k[b, t, hs].astype(np.float64)                       # [H', dk]
            vt = v[b, t, hs].astype(np.float64)                       # [H', dv]
            S = g[:, None, None] * S + kt[:, :, None] * vt[:, None, :]
            qt = q[b, t, hs].astype(np.float64)
            o[b, t] = np.einsum("hd,hde->he", qt, S)
        S_T[n] = S
    return o, S_T


def recurrent_backward(q, k, v, log_g, dO, dS_T=None, S0=None, cu_seqlens=None, heads=None):
    """Gradients of L = sum_t <dO_t, o_t> + sum_n <dS_T[n], S_T[n]> (the
    backward of recurrent_forward for upstream gradients dO and dS_T), fp64.

    dO: [B, T, H, dv]; dS_T: [N, H, dk, dv] or None (zeros). Other arguments
    as recurrent_forward. Returns (dq [B,T,H',dk], dk [B,T,H',dk],
    dv [B,T,H',dv], dlog_g [B,T,H'], dS0 [N,H',dk,dv]), all fp64.

    Per sequence and head, walking t from the last token to the first with
    A = dL/dS_t (starting from dS_T):
        A      += q_t^T dO_t              (o_t = q_t S_t reads S_t)
        dq_t    = dO_t S_t^T
        dk_t    = A v_t^T,  dv_t = k_t A  (S_t gets k_t^T v_t)
        dl_t    = g_t <A, S_{t-1}>        (S_t gets g_t S_{t-1}, g_t = exp(l_t))
        A       = g_t A                   (now dL/dS_{t-1})
    and dS0 = A after the first token. The forward states S_t of one head are
    kept for the walk back.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    log_g = np.asarray(log_g)
    dO = np.asarray(dO)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    hs = np.arange(H) if heads is None else np.asarray(heads, dtype=np.int64)
    bounds = _seq_bounds(B, T, cu_seqlens)
    dq = np.zeros((B, T, len(hs), dk), dtype=np.float64)
    dkk = np.zeros((B, T, len(hs), dk), dtype=np.float64)
    dvv = np.zeros((B, T, len(hs), dv), dtype=np.float64)
    dl = np.zeros((B, T, len(hs)), dtype=np.float64)
    dS0 = np.zeros((len(bounds), len(hs), dk, dv), dtype=np.float64)
    for n, (b, start, end) in enumerate(bounds):
        for i, h in enumerate(hs):
            S = (np.zeros((dk, dv)) if S0 is None
                 else np.asarray(S0)[n, h].astype(np.float64))
            states = [S]  # states[j] = S after j tokens of this sequence
            for t in range(start, end):
                g = np.exp(np.float64(log_g[b, t, h]))
                S = g * S + np.outer(k[b, t, h].astype(np.float64), v[b, t, h].astype(np.float64))
                states.append(S)
            A = (np.zeros((dk, dv)) if dS_T is None
                 else np.asarray(dS_T)[n, h].astype(np.float64))
            for t in range(end - 1, start - 1, -1):
                j = t - start
                qt = q[b, t, h].astype(np.float64)
                kt = k[b, t, h].astype(np.float64)
                vt = v[b, t, h].astype(np.float64)
                dOt = dO[b, t, h].astype(np.float64)
                g = np.exp(np.float64(log_g[b, t, h]))
                A = A + np.outer(qt, dOt)
                dq[b, t, i] = states[j + 1] @ dOt
                dkk[b, t, i] = A @ vt
                dvv[b, t, i] = kt @ A
                dl[b, t, i] = g * np.sum(A * states[j])
                A = g * A
            dS0[n, i] = A
    return dq, dkk, dvv, dl, dS0


def decode_step(q, k, v, log_g, S):
    """One recurrent decode step for a batch of sequences, in fp64.

    q, k: [N, H, dk]; v: [N, H, dv]; log_g: [N, H]; S: [N, H, dk, dv].
    Returns (o [N, H, dv], S' [N, H, dk, dv]) with S' = g S + k^T v and
    o = q S' (the same update and inclusive readout as the forward).
    """
    S = np.asarray(S, dtype=np.float64)
    g = np.exp(np.asarray(log_g, dtype=np.float64))
    kk = np.asarray(k, dtype=np.float64)
    vv = np.asarray(v, dtype=np.float64)
    S_new = g[..., None, None] * S + kk[..., :, None] * vv[..., None, :]
    o = np.einsum("nhd,nhde->nhe", np.asarray(q, dtype=np.float64), S_new)
    return o, S_new


def normwise_error(x, ref) -> float:
    """max_i |x_i - ref_i| / max_i |ref_i|  (the tolerance metric).

    The workloads' tolerance is a maximum relative error; element-wise
    ratios are undefined where the reference is near zero, so the error is
    taken normwise over each output tensor. Non-finite values in x give inf.
    """
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    scale = np.abs(ref).max()
    diff = np.abs(x - ref).max()
    if scale == 0.0:
        return float(diff)
    return float(diff / scale)
