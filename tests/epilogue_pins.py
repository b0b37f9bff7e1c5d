"""Independent checks ("pins") for the token-mixer epilogue.

Each pin takes an implementation
``impl(o, q, k, v, g, a, rms_w, tier, eps) -> z`` over numpy arrays
(o, v, g [R, H, dv]; q, k [R, H, dk]; a [H, dk]; rms_w [n_tiers, dv];
tier [H]) and returns the worst normwise error against a closed form. The
inputs are built so that every intermediate is known exactly: the
self-augmented output o' = o + sigmoid(q . (a * k)) v is made equal to a
chosen c by setting o = c - sigmoid(logit) v for logits whose sigmoid is
exact (0 -> 1/2, ln 3 -> 3/4, -ln 3 -> 1/4); rows of c with entries +-s have
RMS s; and g = +-ln 3 gives silu(g) = 3/4 ln 3 or -1/4 ln 3.

The epilogue is the one of Laplace 3B on AWS Trainium2
(automationscribe.com/?p=7116), "GLA mixer": self-augmentation (a = 0 is a
half-strength skip of the value), Head RMSNorm within each decay tier, SiLU
output gate.
"""
from __future__ import annotations

import math

import numpy as np

LN3 = math.log(3.0)
SILU_LN3 = 0.75 * LN3       # silu(ln 3) = ln 3 * sigmoid(ln 3) = ln 3 * 3/4
SILU_MLN3 = -0.25 * LN3     # silu(-ln 3) = -ln 3 * 1/4


def err(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if x.shape != ref.shape or not np.all(np.isfinite(x)):
        return float("inf")
    s = np.abs(ref).max()
    d = np.abs(x - ref).max()
    return float(d / s) if s > 0 else float(d)


def _signs(rng, shape):
    return np.where(rng.random(shape) < 0.5, -1.0, 1.0)


def _build(rng, R, H, dk, dv, logit_kind, scale=None):
    """Inputs with o' = c known: returns (o, q, k, v, a, c)."""
    v = rng.standard_normal((R, H, dv))
    scale = np.ones(H) if scale is None else np.asarray(scale, np.float64)
    c = _signs(rng, (R, H, dv)) * scale[None, :, None]
    q = rng.standard_normal((R, H, dk))
    k = rng.standard_normal((R, H, dk))
    a = np.zeros((H, dk))
    if logit_kind == "zero":           # a = 0: sigmoid(0) = 1/2
        sig = np.full((R, H, 1), 0.5)
    else:                              # channel 1 only: q_1 a_1 k_1 = +-ln 3
        a[:, 1] = 2.0
        q[:, :, 1] = 1.0
        sgn = _signs(rng, (R, H))
        k[:, :, 1] = sgn * LN3 / 2.0
        sig = np.where(sgn > 0, 0.75, 0.25)[:, :, None]
    o = c - sig * v
    return o, q, k, v, a, c


def _gate(rng, R, H, dv):
    """g = +-ln 3 and silu(g) in closed form."""
    s = _signs(rng, (R, H, dv))
    return s * LN3, np.where(s > 0, SILU_LN3, SILU_MLN3)


def pin_hand_example(impl):
    """Two heads worked by hand (eps = 0).
    Head 0: a = 0, o = (1, 2), v = (4, 4) -> o' = (3, 4), RMS sqrt(12.5);
            tier weight (2, 1); g = (ln 3, 0) -> z = (6 sqrt(2)/5 * 3/4 ln 3, 0).
    Head 1: a = (1, 1), q = (1, 0), k = (ln 3, 5) -> logit ln 3, sigmoid 3/4;
            o = (0, 0), v = (4, -4) -> o' = (3, -3), RMS 3 -> (1, -1);
            tier weight (1, 3); g = (ln 3, -ln 3) -> z = (3/4 ln 3, 3/4 ln 3)."""
    o = np.array([[[1.0, 2.0], [0.0, 0.0]]])
    v = np.array([[[4.0, 4.0], [4.0, -4.0]]])
    q = np.array([[[0.3, -0.7], [1.0, 0.0]]])
    k = np.array([[[0.9, 0.2], [LN3, 5.0]]])
    a = np.array([[0.0, 0.0], [1.0, 1.0]])
    g = np.array([[[LN3, 0.0], [LN3, -LN3]]])
    rms_w = np.array([[2.0, 1.0], [1.0, 3.0]])
    tier = np.array([0, 1])
    want = np.array([[[6.0 * math.sqrt(2.0) / 5.0 * SILU_LN3, 0.0], [SILU_LN3, SILU_LN3]]])
    return err(impl(o, q, k, v, g, a, rms_w, tier, 0.0), want)


def pin_half_skip(impl, seed=0, R=7, H=3, dk=5, dv=8):
    """a = 0 (the page's initialisation): o' = o + v / 2."""
    rng = np.random.default_rng(seed)
    o, q, k, v, a, c = _build(rng, R, H, dk, dv, "zero")
    g, sg = _gate(rng, R, H, dv)
    z = impl(o, q, k, v, g, a, np.ones((1, dv)), np.zeros(H, np.int64), 0.0)
    return err(z, c * sg)


def pin_sigmoid_points(impl, seed=1, R=9, H=2, dk=4, dv=6):
    """Logits +-ln 3 through one key channel scaled by a: sigmoid 3/4 and 1/4."""
    rng = np.random.default_rng(seed)
    o, q, k, v, a, c = _build(rng, R, H, dk, dv, "ln3")
    g, sg = _gate(rng, R, H, dv)
    z = impl(o, q, k, v, g, a, np.ones((1, dv)), np.zeros(H, np.int64), 0.0)
    return err(z, c * sg)


def pin_silu_difference(impl, seed=2, R=5, H=2, dk=3, dv=8):
    """silu(x) - silu(-x) = x: z(g) - z(-g) = y * g for any g."""
    rng = np.random.default_rng(seed)
    o, q, k, v, a, c = _build(rng, R, H, dk, dv, "zero")
    g = rng.standard_normal((R, H, dv)) * 3.0
    w1, t0 = np.ones((1, dv)), np.zeros(H, np.int64)
    d = impl(o, q, k, v, g, a, w1, t0, 0.0) - impl(o, q, k, v, -g, a, w1, t0, 0.0)
    return err(d, c * g)


def pin_eps(impl, seed=3, R=4, H=2, dk=3, dv=16, eps=0.25):
    """eps is added to the mean square under the root: y = c / sqrt(1 + eps)."""
    rng = np.random.default_rng(seed)
    o, q, k, v, a, c = _build(rng, R, H, dk, dv, "zero")
    g, sg = _gate(rng, R, H, dv)
    z = impl(o, q, k, v, g, a, np.ones((1, dv)), np.zeros(H, np.int64), eps)
    return err(z, c * sg / math.sqrt(1.0 + eps))


def pin_scale_invariance(impl, seed=4, R=6, H=4, dk=3, dv=8):
    """Per-head RMS normalisation: rows of +-s (s differs per head) become +-1."""
    rng = np.random.default_rng(seed)
    scale = np.array([0.5, 3.0, 7.0, 0.125])
    o, q, k, v, a, c = _build(rng, R, H, dk, dv, "zero", scale=scale)
    g, sg = _gate(rng, R, H, dv)
    z = impl(o, q, k, v, g, a, np.ones((1, dv)), np.zeros(H, np.int64), 0.0)
    return err(z, np.sign(c) * sg)


def pin_tier_weights(impl, seed=5, R=5, H=6, dk=3, dv=8):
    """Head h uses its tier's weight vector, after normalising on its own
    (heads of one tier have different RMS here)."""
    rng = np.random.default_rng(seed)
    scale = np.array([1.0, 2.0, 4.0, 0.5, 3.0, 1.5])
    o, q, k, v, a, c = _build(rng, R, H, dk, dv, "ln3", scale=scale)
    g, sg = _gate(rng, R, H, dv)
    rms_w = rng.standard_normal((3, dv))
    tier = np.array([2, 0, 1, 2, 0, 1])
    z = impl(o, q, k, v, g, a, rms_w, tier, 0.0)
    return err(z, np.sign(c) * rms_w[tier][None] * sg)


def pin_library_composition(impl, seed=6, R=11, H=3, dk=7, dv=12):
    """Random inputs against torch's own sigmoid, rms_norm and silu (fp64)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    o, v, g = (rng.standard_normal((R, H, dv)) for _ in range(3))
    q, k = (rng.standard_normal((R, H, dk)) for _ in range(2))
    a = rng.standard_normal((H, dk))
    rms_w = rng.standard_normal((2, dv))
    tier = np.array([1, 0, 1])
    T = lambda x: torch.from_numpy(np.asarray(x, np.float64))
    gate = torch.sigmoid((T(q) * T(a)[None] * T(k)).sum(-1, keepdim=True))
    x = T(o) + gate * T(v)
    ref = torch.stack([F.rms_norm(x[:, h], (dv,), T(rms_w[tier[h]]), eps=1e-5) for h in range(H)],
                      dim=1) * F.silu(T(g))
    return err(impl(o, q, k, v, g, a, rms_w, tier, 1e-5), ref.numpy())


ALL_PINS = {
    "hand_example": pin_hand_example,
    "half_skip": pin_half_skip,
    "sigmoid_points": pin_sigmoid_points,
    "silu_difference": pin_silu_difference,
    "eps": pin_eps,
    "scale_invariance": pin_scale_invariance,
    "tier_weights": pin_tier_weights,
    "library_composition": pin_library_composition,
}
