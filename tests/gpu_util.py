"""Helpers for the GPU parity tests: move seeded numpy inputs to the device and
compare HIP results with the fp64 oracle."""
import numpy as np

TOL_BF16 = 2e-3   # max relative (normwise) error, bf16 inputs, fp32 accumulation
TOL_F32 = 1e-5    # fp32 inputs
TOL_BF16_OUT = 2e-3 + 2.0 ** -8  # bf16-rounded output vs the oracle rounded to bf16


# Largest cancellation factor a test may scale the log-gate gradient's bar by.
DG_CANCEL_CAP = 20.0


def dg_cancellation(q, k, dq_ref, dk_ref):
    """How much the log-gate gradient's two dot products cancel. dlog_g is a
    reverse cumulative sum of q.dq - k.dk, so rounding errors of relative size
    e in dq and dk reach it as e * max(1, (|a| + |b|) / |a - b|) with a = q.dq
    and b = k.dk over all tokens (norms over the batch, from the oracle's dq
    and dk in fp64). The factor is printed by the callers and must stay at or
    below DG_CANCEL_CAP: a case that cancels more is too ill-conditioned to
    test at these bars."""
    a = (q.astype(np.float64) * dq_ref).sum(-1)
    b = (k.astype(np.float64) * dk_ref).sum(-1)
    diff = np.linalg.norm(a - b)
    f = 1.0 if diff == 0.0 else max(1.0, (np.linalg.norm(a) + np.linalg.norm(b)) / diff)
    assert f <= DG_CANCEL_CAP, f"dlog_g cancellation factor {f:.1f} above {DG_CANCEL_CAP}"
    return f


def dg_tolerance(tol, q, k, dq_ref, dk_ref):
    """The log-gate gradient's bar: tol times dg_cancellation()."""
    return tol * dg_cancellation(q, k, dq_ref, dk_ref)


def _normwise(x, ref):
    scale = np.abs(ref).max() if ref.size else 0.0
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    diff = np.abs(x - ref).max()
    return float(diff if scale == 0.0 else diff / scale)


def tok_error(x, ref, cu=None):
    """Largest normwise error over (sequence, head) pairs of a token-major
    tensor [B, T, H, ...] (outputs, per-token gradients): each pair's error
    is max |x - ref| / max |ref| over that sequence's tokens and that head's
    channels, so a head of small magnitude is held to the same relative bar
    as a large one. With cu (packed batch, B = 1) the sequences are the
    spans cu[n] .. cu[n+1]."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    worst = 0.0
    if cu is None:
        spans = [(b, 0, x.shape[1]) for b in range(x.shape[0])]
    else:
        spans = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    for b, s, e in spans:
        if e <= s:
            continue
        for h in range(x.shape[2]):
            worst = max(worst, _normwise(x[b, s:e, h], ref[b, s:e, h]))
    return worst


def state_error(x, ref):
    """Largest normwise error over (sequence, head) pairs of a state tensor
    [N, H, ...]."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    worst = 0.0
    for n in range(x.shape[0]):
        for h in range(x.shape[1]):
            worst = max(worst, _normwise(x[n, h], ref[n, h]))
    return worst


def dev(x, dtype=None):
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def in_dtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def host(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def say(msg):
    print(msg, flush=True)


def grad_errors(got, ref, cu=None):
    """Errors of the backward's five gradients (dq, dk, dv, dlog_g, dS0)
    against the oracle: per (sequence, head) pair for dq, dk, dv and dS0;
    dlog_g normwise over the whole tensor. dlog_g is a reverse cumulative sum
    of q.dq - k.dk, a difference of two dot products, so within one pair its
    relative error is amplified by how much the two cancel there (about 26x
    on a one-token sequence); its per-pair error is returned as the sixth
    value, for the log."""
    errs = [tok_error(g, r, cu) for g, r in zip(got[:3], ref[:3])]
    errs.append(_normwise(np.asarray(got[3], np.float64), np.asarray(ref[3], np.float64)))
    errs.append(state_error(got[4], ref[4]))
    errs.append(tok_error(got[3], ref[3], cu))
    return errs
