"""GPU parity of the token-mixer epilogue (gla_mixer_epilogue) against the fp64 oracle.

The epilogue of Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116),
"GLA mixer": self-augmentation o' = o + sigmoid(q.(a*k)) v, the head's RMSNorm
with its decay tier's weights, and the SiLU output gate. Tolerances: 1e-5
normwise for fp32 results (the kernel computes in fp32), 2e-3 + 2^-8 for a
bf16 output compared with the oracle rounded to bf16.
"""
import numpy as np
import pytest

import gpu_util as gu
from gated_linear_attention_amd import synth
from oracle import c_oracle
from oracle import epilogue_oracle as eo
from oracle import gla_oracle as orc

pytestmark = pytest.mark.gpu

DIMS = [(64, 64), (64, 128), (128, 64), (128, 128), (96, 192)]


def run(o, q, k, v, g, a, tier_w, tier, eps, o_dtype=None, in_dtype=None, out_dtype=None,
        in_place=False):
    import torch
    import gated_linear_attention_amd as gla
    to = gu.dev(o, o_dtype)
    ti = lambda x: gu.dev(x, in_dtype)
    w = gla.head_rms_weights(gu.dev(tier_w), gu.dev(tier))
    z = gla.mixer_epilogue(to, ti(q), ti(k), ti(v), ti(g), gu.dev(a), w, eps,
                           out_dtype=out_dtype, z=to if in_place else None)
    torch.cuda.synchronize()
    return gu.host(z)


@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("n_tok", [1, 37])
def test_epilogue_bf16_inputs(dk, dv, n_tok):
    """bf16 q, k, v, g, fp32 o and z; row counts that leave partial workgroups."""
    gu.say(f"epilogue dk={dk} dv={dv} n_tok={n_tok}")
    H = 3
    o, q, k, v, g = synth.make_epilogue_inputs(n_tok, H, dk, dv, seed=51)
    a, tw, tier = synth.make_epilogue_params(H, dk, dv, seed=52, n_tiers=2)
    z = run(o, q, k, v, g, a, tw, tier, 1e-6)
    ref = eo.mixer_epilogue(o, q, k, v, g, a, tw, tier, 1e-6)
    e = orc.normwise_error(z, ref)
    gu.say(f"   z err {e:.2e}")
    assert e <= 1e-5, e


@pytest.mark.parametrize("o_dt,in_dt,out_dt", [("f32", "f32", "f32"), ("bf16", "bf16", "bf16"),
                                               ("bf16", "f32", "f32"), ("f32", "bf16", "bf16")])
def test_epilogue_dtypes(o_dt, in_dt, out_dt):
    import torch
    gu.say(f"epilogue dtypes o={o_dt} in={in_dt} out={out_dt}")
    dk, dv, H, n_tok = 96, 192, 16, 50
    o, q, k, v, g = synth.make_epilogue_inputs(n_tok, H, dk, dv, seed=53, dtype=in_dt)
    if o_dt == "bf16":
        o = synth.round_bf16(o)
    a, tw, tier = synth.make_epilogue_params(H, dk, dv, seed=54)
    T = lambda s: torch.bfloat16 if s == "bf16" else torch.float32
    z = run(o, q, k, v, g, a, tw, tier, 1e-5, o_dtype=T(o_dt), in_dtype=T(in_dt),
            out_dtype=T(out_dt))
    ref = eo.mixer_epilogue(o, q, k, v, g, a, tw, tier, 1e-5)
    if out_dt == "bf16":
        ref = synth.round_bf16(ref.astype(np.float32))
    e = orc.normwise_error(z, ref)
    gu.say(f"   z err {e:.2e}")
    assert e <= (gu.TOL_BF16_OUT if out_dt == "bf16" else 1e-5), e


def test_epilogue_half_skip_and_in_place():
    """a = 0 (the page's initialisation: o' = o + v/2), z written over o."""
    gu.say("epilogue a = 0, in place")
    dk, dv, H, n_tok = 128, 128, 4, 33
    o, q, k, v, g = synth.make_epilogue_inputs(n_tok, H, dk, dv, seed=55)
    a, tw, tier = synth.make_epilogue_params(H, dk, dv, seed=56, a_std=0.0)
    z = run(o, q, k, v, g, a, tw, tier, 1e-6, in_place=True)
    ref = eo.mixer_epilogue(o, q, k, v, g, a, tw, tier, 1e-6)
    assert orc.normwise_error(z, ref) <= 1e-5


def test_epilogue_after_laplace_forward():
    """laplace_2k end to end: the fixed-decay forward, then the epilogue with
    4 tiers of 4 heads; the oracle runs its forward and its epilogue over every
    head, and each (sequence, head) pair is held to its own normwise bar."""
    import torch
    import gated_linear_attention_amd as gla
    gu.say("laplace_2k forward + epilogue")
    w = synth.WORKLOADS["laplace_2k"]
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    gate = synth.make_epilogue_inputs(w.B * w.T, w.H, w.dk, w.dv, seed=57)[4]
    gate = gate.reshape(w.B, w.T, w.H, w.dv)
    a, tw, tier = synth.make_epilogue_params(w.H, w.dk, w.dv, seed=58)
    bf = lambda x: gu.dev(x, torch.bfloat16)
    tq, tk, tv = bf(q), bf(k), bf(v)
    o, _ = gla.fwd_chunked_fixed_decay(tq, tk, tv, gu.dev(synth.fixed_log_decays(w.H)),
                                       output_final_state=False)
    z = gla.mixer_epilogue(o, tq, tk, tv, bf(gate), gu.dev(a),
                           gla.head_rms_weights(gu.dev(tw), gu.dev(tier)), 1e-6,
                           out_dtype=torch.bfloat16)
    z = gu.host(z)
    o_ref, _, _ = c_oracle.fwd(q, k, v, lg, None, None, nthreads=16)
    z_ref = eo.mixer_epilogue(o_ref, q, k, v, gate, a, tw, tier, 1e-6)
    z_ref = synth.round_bf16(z_ref.astype(np.float32))
    e = gu.tok_error(z, z_ref)
    gu.say(f"   z err {e:.2e}")
    assert e <= gu.TOL_BF16_OUT, e
