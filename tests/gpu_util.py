"""Helpers for the GPU parity tests: move seeded numpy inputs to the device and
compare HIP results with the fp64 oracle."""
import numpy as np

TOL_BF16 = 2e-3   # max relative (normwise) error, bf16 inputs, fp32 accumulation
TOL_F32 = 1e-5    # fp32 inputs
TOL_BF16_OUT = 2e-3 + 2.0 ** -8  # bf16-rounded output vs the oracle rounded to bf16


def dg_tolerance(tol, q, k, dq_ref, dk_ref):
    """Bar for the log-gate gradient. It is a reverse cumulative sum of
    q.dq - k.dk, a difference of two dot products, so rounding errors of the
    size `tol` in dq and dk reach it multiplied by how much the two cancel:
    tol * max(1, (|a| + |b|) / |a - b|) with a = q.dq and b = k.dk over all
    tokens (norms over the batch, from the oracle's dq and dk in fp64)."""
    a = (q.astype(np.float64) * dq_ref).sum(-1)
    b = (k.astype(np.float64) * dk_ref).sum(-1)
    diff = np.linalg.norm(a - b)
    if diff == 0.0:
        return tol
    return tol * max(1.0, (np.linalg.norm(a) + np.linalg.norm(b)) / diff)


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
