"""fp64 CPU oracle for the token-mixer epilogue around the GLA readout.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module: only the tests, the package's smoke check and the benchmark's
CPU-baseline leg do. It shares no code with the HIP path.

Source: Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), section
"GLA mixer". After the state readout o_t of a head, the page adds a gated copy
of the value (self-augmentation): the gate is the sigmoid of the query dotted
with a learned per-channel rescaling a of the key, and a = 0 at
initialisation gives a half-strength skip of the value. The per-head outputs
then pass through a Head RMSNorm inside each decay tier, are concatenated and
gated by SiLU of the gate stream g_t (the output projection that follows is
a dense layer with trained weights, not part of this epilogue). The page's
equation images are lost; the readings taken here:
  * self-augmentation: o'_t = o_t + sigmoid(sum_i q_i a_i k_i) v_t, with a
    per head and key channel (a[h, i]);
  * Head RMSNorm: each head's d_v outputs are normalised on their own,
    y = o' / sqrt(mean_j o'_j^2 + eps), then scaled by the weight vector of
    the head's tier (heads of one tier share it);
  * output gate: z = y * silu(g), silu(x) = x * sigmoid(x), with g the head's
    d_v slice of the gate stream (the concatenation is the [.., H, d_v]
    layout itself).
Pins: tests/test_oracle_epilogue.py (a hand-worked example, the page's
a = 0 half skip, sigmoid symmetry, the SiLU difference identity, unit RMS,
scale invariance, tier selection) and its planted mutants.
"""
from __future__ import annotations

import numpy as np

__all__ = ["mixer_epilogue", "sigmoid", "silu"]


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def mixer_epilogue(o, q, k, v, g, a, rms_w, tier, eps, parts=False):
    """The epilogue in fp64, in the page's order.

    o, v, g: [..., H, dv]; q, k: [..., H, dk]; a: [H, dk]; rms_w: [n_tiers, dv];
    tier: [H] tier index of each head; eps: RMSNorm epsilon.
    Returns z [..., H, dv]; with parts=True also (o_aug, y).
    """
    o = np.asarray(o, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(rms_w, dtype=np.float64)[np.asarray(tier, dtype=np.int64)]  # [H, dv]
    # 1. self-augmentation: gate = sigmoid(q . (a * k)) per (token, head)
    logit = np.sum(q * a * k, axis=-1, keepdims=True)
    o_aug = o + sigmoid(logit) * v
    # 2. Head RMSNorm over each head's dv channels, tier-shared weights
    ms = np.mean(o_aug * o_aug, axis=-1, keepdims=True)
    y = o_aug / np.sqrt(ms + eps) * w
    # 3. SiLU output gate
    z = y * silu(g)
    return (z, o_aug, y) if parts else z
