"""GPU parity of the serving-pool decode step (gla_decode_step_slots).

Request n decodes against pool entry slots[n] (Laplace 3B on AWS Trainium2,
"Inference optimization": one fixed-size state per sequence in the serving
engine's pool, fixed-width padded batches). Pins: each valid lane equals the
oracle's decode step on the gathered state; padded lanes (slots outside
[0, P)) output zeros; pool entries no request names are bit-for-bit unchanged.
"""
import numpy as np
import pytest

import gpu_util as gu
from gated_linear_attention_amd import synth
from oracle import gla_oracle as orc

pytestmark = pytest.mark.gpu


def run_slots(P, H, dk, dv, slots, dtype, out_dtype=None, seed=3, steps=2):
    import torch
    import gated_linear_attention_amd as gla
    N = len(slots)
    pool = synth.make_decode_state(P, H, dk, dv, seed=seed)
    ref = pool.astype(np.float64).copy()
    S = gu.dev(pool)
    sl = gu.dev(np.asarray(slots, dtype=np.int32))
    valid = [n for n, s in enumerate(slots) if 0 <= s < P]
    worst_o = 0.0
    for step in range(steps):
        q, k, v, lg = synth.make_decode_step_inputs(N, H, dk, dv, seed=5000 + step, dtype=dtype)
        td = gu.in_dtype(dtype)
        o = gla.decode_step_slots(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lg), S, sl,
                                  out_dtype=out_dtype)
        o = gu.host(o)
        o_ref = np.zeros((N, H, dv))
        if valid:
            idx = [slots[n] for n in valid]
            o_v, S_v = orc.decode_step(q[valid], k[valid], v[valid], lg[valid], ref[idx])
            o_ref[valid] = o_v
            ref[idx] = S_v
        if out_dtype == torch.bfloat16:
            o_ref = synth.round_bf16(o_ref.astype(np.float32))
        pad = [n for n in range(N) if n not in valid]
        assert np.all(o[pad] == 0.0)
        worst_o = max(worst_o, orc.normwise_error(o, o_ref))
    S_gpu = gu.host(S)
    touched = sorted({slots[n] for n in valid})
    untouched = [p for p in range(P) if p not in touched]
    np.testing.assert_array_equal(S_gpu[untouched], pool[untouched].astype(np.float64))
    eS = orc.normwise_error(S_gpu[touched], ref[touched]) if touched else 0.0
    return worst_o, eS


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128), (96, 192)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_slots_match_dense_on_gathered_states(dk, dv, dtype):
    gu.say(f"decode slots dk={dk} dv={dv} {dtype}")
    eo, eS = run_slots(P=10, H=3, dk=dk, dv=dv, slots=[3, -1, 7, 0, -1, 9], dtype=dtype)
    gu.say(f"   o err {eo:.2e}  S err {eS:.2e}")
    assert eo <= 1e-5 and eS <= 1e-6


@pytest.mark.parametrize("dk,dv", [(128, 128), (96, 192)])
def test_slots_many_requests(dk, dv):
    """200 requests x 3 heads (one workgroup per pair) on a 300-entry pool,
    every fifth lane padded."""
    gu.say(f"decode slots, 200 requests dk={dk} dv={dv}")
    rng = np.random.default_rng(9)
    slots = [int(x) for x in rng.permutation(300)[:200]]
    slots = [-1 if n % 5 == 4 else s for n, s in enumerate(slots)]
    eo, eS = run_slots(P=300, H=3, dk=dk, dv=dv, slots=slots, dtype="bf16")
    gu.say(f"   o err {eo:.2e}  S err {eS:.2e}")
    assert eo <= 1e-5 and eS <= 1e-6


def test_slots_out_of_range_are_padding():
    gu.say("decode slots out of range")
    eo, eS = run_slots(P=6, H=2, dk=128, dv=128, slots=[6, -5, 2, 1000, 5], dtype="bf16")
    assert eo <= 1e-5 and eS <= 1e-6


def test_slots_bf16_output():
    import torch
    gu.say("decode slots bf16 output")
    eo, eS = run_slots(P=9, H=2, dk=128, dv=128, slots=[8, 1, -1, 4], dtype="bf16",
                       out_dtype=torch.bfloat16)
    assert eo <= gu.TOL_BF16_OUT and eS <= 1e-6


def test_slots_all_padding_and_permuted_pool():
    gu.say("decode slots: all padded; then a permutation of a larger pool")
    eo, eS = run_slots(P=4, H=2, dk=64, dv=64, slots=[-1, -1, -1], dtype="bf16")
    assert eo == 0.0 and eS == 0.0
    rng = np.random.default_rng(17)
    slots = list(rng.permutation(96)[:80])
    slots[5] = slots[40] = -1
    eo, eS = run_slots(P=96, H=4, dk=128, dv=128, slots=slots, dtype="bf16", steps=3)
    assert eo <= 1e-5 and eS <= 1e-6
