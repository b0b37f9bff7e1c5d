"""GPU parity of the fused decode step + mixer epilogue (gla_decode_mixer).

Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), "GLA mixer": one
recurrent step S <- exp(l) S + k^T v, o = q S, then o' = o + sigmoid(q.(a*k)) v,
the head's RMSNorm with its tier weights and the SiLU output gate. Checked
against the fp64 oracle's decode step followed by its epilogue, with a dense
state and with a slot-indexed pool (padded lanes give z = 0 and touch no
state; untouched pool entries stay bit-identical).
"""
import numpy as np
import pytest

import gpu_util as gu
from gated_linear_attention_amd import synth
from oracle import epilogue_oracle as eo
from oracle import gla_oracle as orc

pytestmark = pytest.mark.gpu

DIMS = [(128, 128), (64, 64), (128, 64), (64, 128), (96, 192)]


def _run(N, H, dk, dv, slots=None, P=None, steps=2, dtype="bf16", out_bf16=False, seed=0):
    import torch
    import gated_linear_attention_amd as gla
    n_state = N if slots is None else P
    S_np = synth.make_decode_state(n_state, H, dk, dv, seed=70 + seed)
    ref = S_np.astype(np.float64).copy()
    S = gu.dev(S_np)
    a, tw, tier = synth.make_epilogue_params(H, dk, dv, seed=71 + seed, n_tiers=2)
    w = gla.head_rms_weights(gu.dev(tw), gu.dev(tier))
    sl = None if slots is None else gu.dev(np.asarray(slots, np.int32))
    valid = list(range(N)) if slots is None else [n for n, s in enumerate(slots) if 0 <= s < P]
    idx = valid if slots is None else [slots[n] for n in valid]
    td = gu.in_dtype(dtype)
    worst = 0.0
    for step in range(steps):
        q, k, v, lg = synth.make_decode_step_inputs(N, H, dk, dv, seed=600 + 10 * seed + step,
                                                    dtype=dtype)
        gout = synth.make_epilogue_inputs(N, H, dk, dv, seed=700 + step, dtype=dtype)[4]
        z = gla.decode_mixer(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lg), S,
                             gu.dev(gout, td), gu.dev(a), w, 1e-6, slots=sl,
                             out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
        z = gu.host(z)
        z_ref = np.zeros((N, H, dv))
        if valid:
            o_v, S_v = orc.decode_step(q[valid], k[valid], v[valid], lg[valid], ref[idx])
            ref[idx] = S_v
            z_ref[valid] = eo.mixer_epilogue(o_v, q[valid], k[valid], v[valid], gout[valid], a, tw,
                                             tier, 1e-6)
        if out_bf16:
            z_ref = synth.round_bf16(z_ref.astype(np.float32))
        pad = [n for n in range(N) if n not in valid]
        assert np.all(z[pad] == 0.0)
        worst = max(worst, orc.normwise_error(z, z_ref))
    S_gpu = gu.host(S)
    eS = orc.normwise_error(S_gpu[idx], ref[idx]) if idx else 0.0
    untouched = sorted(set(range(n_state)) - set(idx))
    np.testing.assert_array_equal(S_gpu[untouched], S_np[untouched].astype(np.float64))
    return worst, eS


@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("N", [37, 200])
def test_decode_mixer_dense(dk, dv, N):
    gu.say(f"decode+epilogue dense dk={dk} dv={dv} N={N}")
    ez, eS = _run(N, 3, dk, dv)
    gu.say(f"   z err {ez:.2e}  S err {eS:.2e}")
    assert ez <= 1e-5 and eS <= 1e-6, (ez, eS)


@pytest.mark.parametrize("dk,dv", [(128, 128), (96, 192)])
def test_decode_mixer_slots(dk, dv):
    """A 40-entry pool, 12 requests, three padded lanes (-1 and out of range)."""
    gu.say(f"decode+epilogue slots dk={dk} dv={dv}")
    slots = [5, -1, 17, 0, 39, 40, 8, 22, -7, 31, 2, 11]
    ez, eS = _run(len(slots), 4, dk, dv, slots=slots, P=40, seed=1)
    gu.say(f"   z err {ez:.2e}  S err {eS:.2e}")
    assert ez <= 1e-5 and eS <= 1e-6, (ez, eS)


def test_decode_mixer_bf16_io():
    gu.say("decode+epilogue bf16 in/out")
    ez, eS = _run(50, 16, 96, 192, out_bf16=True, seed=2)
    assert ez <= gu.TOL_BF16_OUT and eS <= 1e-6, (ez, eS)


def test_decode_mixer_f32_inputs():
    gu.say("decode+epilogue fp32 inputs")
    ez, eS = _run(30, 2, 128, 128, dtype="f32", seed=3)
    assert ez <= 1e-5 and eS <= 1e-6, (ez, eS)
