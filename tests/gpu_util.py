"""Helpers for the GPU parity tests: move seeded numpy inputs to the device and
compare HIP results with the fp64 oracle."""
import numpy as np

TOL_BF16 = 2e-3   # max relative (normwise) error, bf16 inputs, fp32 accumulation
TOL_F32 = 1e-5    # fp32 inputs
TOL_BF16_OUT = 2e-3 + 2.0 ** -8  # bf16-rounded output vs the oracle rounded to bf16


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
