"""GPU parity of the decode step (gla_decode_step) against the fp64 oracle.

The oracle's decode_step is the recurrence S <- exp(l) S + k^T v, o = q S of
Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), "GLA mixer".
"""
import numpy as np
import pytest

import gpu_util as gu
from gated_linear_attention_amd import synth
from oracle import c_oracle
from oracle import gla_oracle as orc

pytestmark = pytest.mark.gpu


def _run_chain(N, H, dk, dv, steps, dtype, out_dtype, seed=7, state_steps=None):
    """Chained decode steps on the GPU and in the C oracle over every
    (sequence, head) pair: the largest per-pair normwise error of o over all
    steps, and of the state after the steps in state_steps (default: the
    first and the last; the state is copied back only there)."""
    import torch
    import gated_linear_attention_amd as gla
    S_np = synth.make_decode_state(N, H, dk, dv, seed=seed)
    S = gu.dev(S_np)
    S_ref = S_np.astype(np.float64)
    del S_np
    state_steps = (0, steps - 1) if state_steps is None else state_steps
    worst_o, worst_S = 0.0, 0.0
    for s in range(steps):
        q, k, v, lg = synth.make_decode_step_inputs(N, H, dk, dv, seed=4000 + s, dtype=dtype)
        o = gla.decode_step(gu.dev(q, gu.in_dtype(dtype)), gu.dev(k, gu.in_dtype(dtype)),
                            gu.dev(v, gu.in_dtype(dtype)), gu.dev(lg), S, out_dtype=out_dtype)
        o_ref, _ = c_oracle.decode(q, k, v, lg, S_ref, nthreads=16)
        o_gpu = gu.host(o)
        if out_dtype == torch.bfloat16:
            o_ref = synth.round_bf16(o_ref.astype(np.float32))
        worst_o = max(worst_o, gu.state_error(o_gpu, o_ref))
        if s in state_steps:
            worst_S = max(worst_S, gu.state_error(S.cpu().numpy(), S_ref))
    return worst_o, worst_S


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128), (96, 192)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N", [37, 200])
def test_decode_small(dk, dv, dtype, N):
    """37 x 3 pairs run as column slices (fewer than two pairs per CU), 200 x 3
    with one workgroup per pair."""
    import torch
    gu.say(f"decode dk={dk} dv={dv} {dtype} N={N}")
    eo, eS = _run_chain(N=N, H=3, dk=dk, dv=dv, steps=4, dtype=dtype, out_dtype=torch.float32)
    tol = gu.TOL_BF16 if dtype == "bf16" else gu.TOL_F32
    assert eo <= tol and eS <= tol, (eo, eS)
    assert eo <= 1e-5 and eS <= 1e-6  # fp32 arithmetic on exact inputs


def test_decode_bf16_output():
    import torch
    gu.say("decode bf16 output")
    eo, eS = _run_chain(N=16, H=4, dk=128, dv=128, steps=3, dtype="bf16", out_dtype=torch.bfloat16)
    assert eo <= gu.TOL_BF16_OUT and eS <= 1e-6, (eo, eS)


def test_decode_reset_and_unit_gate():
    import torch
    import gated_linear_attention_amd as gla
    gu.say("decode reset / unit gate")
    N, H, d = 5, 2, 64
    S_np = synth.make_decode_state(N, H, d, d, seed=1)
    q, k, v, _ = synth.make_decode_step_inputs(N, H, d, d, seed=2)
    for lgv in (-np.inf, 0.0, -30.0):
        lg = np.full((N, H), lgv, np.float32)
        S = gu.dev(S_np)
        o = gla.decode_step(gu.dev(q, torch.bfloat16), gu.dev(k, torch.bfloat16),
                            gu.dev(v, torch.bfloat16), gu.dev(lg), S)
        o_ref, S_ref = orc.decode_step(q, k, v, lg, S_np)
        assert orc.normwise_error(gu.host(o), o_ref) <= 1e-6
        assert orc.normwise_error(gu.host(S), S_ref) <= 1e-6


def test_decode_full_size_100_steps():
    """1,280 sequences x 16 heads, d = 128, fp32 state (1.34 GB) updated in place
    over 100 chained steps: every (sequence, head) pair's output at every step,
    and every pair's state after steps 1 and 100."""
    import torch
    gu.say("decode full size, 100 chained steps")
    D = synth.DECODE
    eo, eS = _run_chain(D["N"], D["H"], D["dk"], D["dv"], D["steps"], "bf16", torch.float32,
                        seed=D["state_seed"])
    gu.say(f"   o err {eo:.2e}  S err {eS:.2e} (max over 20,480 pairs)")
    assert eo <= gu.TOL_BF16 and eS <= gu.TOL_BF16, (eo, eS)
    assert eo <= 1e-5 and eS <= 1e-5, (eo, eS)
