"""Seeded synthetic inputs for the gated linear-attention workloads.

This module is the only code shared by the fp64 oracle's tests and the HIP
path's tests and benchmark. It draws random numbers and rounds them to the
storage precision; it holds none of the method's arithmetic (no state update,
no readout, no decay products).

Recipe (one GLA layer, H heads, synthetic data, no trained weights):
  * q, v ~ N(0, 1); k ~ N(0, 1) / sqrt(d_k)  (the 1/sqrt(d_k) of scaled
    attention is folded into k, so the method itself applies no scale);
  * log-gates  l = logsigmoid(N(0, 1) + bias)  with bias 3 (4 for the
    long-context prefill), one scalar per (token, head): "simple" GLA;
  * initial states S0 ~ N(0, 0.02^2) where a workload has one;
  * bf16 tensors are drawn in fp32 and rounded to bf16 with
    round-to-nearest-even, so the oracle reads exactly the values the GPU
    reads; log-gates are computed in fp64 and stored as fp32.

Every generator is driven by ``numpy.random.default_rng(seed)`` with a fixed
draw order (lengths, q, k, v, gate pre-activation, S0).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "round_bf16",
    "log_sigmoid",
    "Workload",
    "WORKLOADS",
    "make_forward_inputs",
    "make_decode_state",
    "make_decode_step_inputs",
    "varlen_lengths",
    "laplace_decay_schedule",
    "fixed_log_decays",
    "make_epilogue_params",
    "make_epilogue_inputs",
]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns float32 values that are exactly representable in bf16, so a later
    ``.to(torch.bfloat16)`` is exact. NaN stays NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def log_sigmoid(x: np.ndarray) -> np.ndarray:
    """log(1 / (1 + exp(-x))) in fp64, stable for large |x|."""
    x = np.asarray(x, dtype=np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype and distributions."""

    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: str            # "f32" or "bf16" for q, k, v
    gate_bias: float      # log g = logsigmoid(N(0,1) + gate_bias)
    s0_std: float         # 0 -> no initial state (S0 = NULL)
    chunk: int            # chunk size the workload names
    num_seqs: int = 0     # >0: varlen packed batch of this many sequences
    len_lo: int = 0
    len_hi: int = 0
    seed: int = 0
    fixed_decay: bool = False  # log g[b, t, h] = ln(lambda_h) of the geometric schedule


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", B=1, T=256, H=2, dk=64, dv=64, dtype="f32",
                         gate_bias=3.0, s0_std=0.0, chunk=64, seed=1000),
    "train_2k": Workload("train_2k", B=8, T=2048, H=16, dk=128, dv=128, dtype="bf16",
                         gate_bias=3.0, s0_std=0.0, chunk=128, seed=1001),
    "prefill_64k": Workload("prefill_64k", B=1, T=65536, H=32, dk=128, dv=128, dtype="bf16",
                            gate_bias=4.0, s0_std=0.02, chunk=64, seed=1002),
    "varlen_64": Workload("varlen_64", B=1, T=0, H=16, dk=128, dv=128, dtype="bf16",
                          gate_bias=3.0, s0_std=0.02, chunk=128, num_seqs=64,
                          len_lo=128, len_hi=8192, seed=1004),
    # Laplace 3B's mixer shape: 16 heads of d_k = 96, d_v = 192 with the
    # fixed geometric decays, 8 sequences of 2,048 tokens.
    "laplace_2k": Workload("laplace_2k", B=8, T=2048, H=16, dk=96, dv=192, dtype="bf16",
                           gate_bias=0.0, s0_std=0.0, chunk=64, seed=1005, fixed_decay=True),
}

# Batched decode: 1,280 sequences x 16 heads, d_k = d_v = 128, fp32 state
# updated in place over 100 chained steps.
DECODE = dict(N=1280, H=16, dk=128, dv=128, steps=100, state_seed=1003,
              step_seed_base=4000, gate_bias=3.0, s0_std=0.02)


def varlen_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """n i.i.d. integer lengths, uniform on [lo, hi] inclusive."""
    return rng.integers(lo, hi + 1, size=n, dtype=np.int64)


def _normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def make_forward_inputs(w: Workload, *, seed: int | None = None, B: int | None = None,
                        T: int | None = None, H: int | None = None,
                        lengths=None):
    """Draw (q, k, v, log_g, S0, cu_seqlens) for a chunked-forward workload.

    Shapes: q, k [B, T, H, dk]; v [B, T, H, dv]; log_g [B, T, H] fp32;
    S0 [N, H, dk, dv] fp32 or None; cu_seqlens int32 [N+1] or None.
    A varlen workload packs its sequences into B = 1 rows of length
    sum(lengths). Overrides (B, T, H, lengths) shrink a workload while keeping
    its distributions; values are fp32 arrays holding bf16-exact numbers when
    the workload's dtype is bf16.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    H = w.H if H is None else H
    cu = None
    if w.num_seqs or lengths is not None:
        if lengths is None:
            lengths = varlen_lengths(rng, w.num_seqs, w.len_lo, w.len_hi)
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B, T, N = 1, int(cu[-1]), len(lengths)
    else:
        B = w.B if B is None else B
        T = w.T if T is None else T
        N = B
    q = _store(_normal(rng, (B, T, H, w.dk)), w.dtype)
    k = _store(_normal(rng, (B, T, H, w.dk), 1.0 / math.sqrt(w.dk)), w.dtype)
    v = _store(_normal(rng, (B, T, H, w.dv)), w.dtype)
    pre = rng.standard_normal(size=(B, T, H)) + w.gate_bias
    log_g = log_sigmoid(pre).astype(np.float32)
    if w.fixed_decay:
        log_g = np.ascontiguousarray(
            np.broadcast_to(fixed_log_decays(H), (B, T, H)), dtype=np.float32)
    S0 = None
    if w.s0_std > 0:
        S0 = _normal(rng, (N, H, w.dk, w.dv), w.s0_std)
    return q, k, v, log_g, S0, cu


def make_backward_grads(w: Workload, B: int, T: int, H: int, N: int, *, seed: int,
                        final_state: bool = True, s_std: float = 0.02):
    """Upstream gradients for a backward run: dO [B, T, H, dv] ~ N(0, 1) in the
    workload's dtype (bf16-exact values when bf16), and dS_T [N, H, dk, dv]
    ~ N(0, s_std^2) fp32 (None when final_state is False)."""
    rng = np.random.default_rng(seed)
    dO = _store(_normal(rng, (B, T, H, w.dv)), w.dtype)
    dS_T = _normal(rng, (N, H, w.dk, w.dv), s_std) if final_state else None
    return dO, dS_T


def make_decode_state(N: int, H: int, dk: int, dv: int, *, seed: int, std: float = 0.02):
    """Initial fp32 decode state S[N, H, dk, dv] ~ N(0, std^2)."""
    rng = np.random.default_rng(seed)
    return _normal(rng, (N, H, dk, dv), std)


def make_decode_step_inputs(N: int, H: int, dk: int, dv: int, *, seed: int,
                            dtype: str = "bf16", gate_bias: float = 3.0):
    """One decode step's (q, k, v, log_g): q, k [N, H, dk]; v [N, H, dv]; log_g [N, H]."""
    rng = np.random.default_rng(seed)
    q = _store(_normal(rng, (N, H, dk)), dtype)
    k = _store(_normal(rng, (N, H, dk), 1.0 / math.sqrt(dk)), dtype)
    v = _store(_normal(rng, (N, H, dv)), dtype)
    log_g = log_sigmoid(rng.standard_normal(size=(N, H)) + gate_bias).astype(np.float32)
    return q, k, v, log_g


def fixed_log_decays(H: int) -> np.ndarray:
    """The schedule's ln(lambda_h) for H heads as the fp32 values a fixed-decay
    forward takes (shape [H])."""
    return laplace_decay_schedule(H=H).astype(np.float32)


def laplace_decay_schedule(H: int = 16, t_min: float = 1.0, t_max: float = 2048.0) -> np.ndarray:
    """Fixed per-head decays of the Laplace 3B GLA mixer, as log-gates.

    Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), "Decay
    schedule": decays are fixed at initialisation on a geometric schedule
    between T_min = 1 and T_max = 2048 tokens; head 0 has half-life 1
    (lambda_0 = 0.5) and head 15 half-life 2048 (lambda_15 ~ 0.9997). The
    equations themselves are lost from the page; the reading taken here is a
    geometric spread of half-lives, half_life_h = T_min (T_max/T_min)^(h/(H-1)),
    with lambda_h = 2^(-1/half_life_h); a single head (H = 1) takes T_min.
    Returns ln(lambda_h), shape [H], fp64.
    """
    h = np.arange(H, dtype=np.float64)
    frac = h / (H - 1) if H > 1 else np.zeros(H)
    half_life = t_min * (t_max / t_min) ** frac
    return -np.log(2.0) / half_life


def make_epilogue_params(H: int, dk: int, dv: int, *, seed: int, n_tiers: int = 4,
                         a_std: float = 0.1):
    """Mixer-epilogue parameters: a [H, dk] ~ N(0, a_std^2) fp32 (0 at the
    page's initialisation; a_std = 0 gives that), tier weights [n_tiers, dv]
    ~ 1 + N(0, 0.1^2) fp32, and tier [H]: consecutive groups of H / n_tiers
    heads."""
    rng = np.random.default_rng(seed)
    a = _normal(rng, (H, dk), a_std) if a_std > 0 else np.zeros((H, dk), np.float32)
    tier_w = (1.0 + _normal(rng, (n_tiers, dv), 0.1)).astype(np.float32)
    tier = (np.arange(H) * n_tiers // H).astype(np.int32)
    return a, tier_w, tier


def make_epilogue_inputs(n_tok: int, H: int, dk: int, dv: int, *, seed: int,
                         dtype: str = "bf16"):
    """(o, q, k, v, g) for an epilogue call on n_tok tokens: o [n_tok, H, dv]
    ~ N(0, 1) fp32 (a readout); q, k, v as the forward's; g (gate stream)
    ~ N(0, 1), in `dtype`."""
    rng = np.random.default_rng(seed)
    o = _normal(rng, (n_tok, H, dv))
    q = _store(_normal(rng, (n_tok, H, dk)), dtype)
    k = _store(_normal(rng, (n_tok, H, dk), 1.0 / math.sqrt(dk)), dtype)
    v = _store(_normal(rng, (n_tok, H, dv)), dtype)
    g = _store(_normal(rng, (n_tok, H, dv)), dtype)
    return o, q, k, v, g

