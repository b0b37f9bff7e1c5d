"""GPU parity of the chunked backward (gla_bwd_chunked) against the fp64
oracle's backward (the reverse-mode adjoint of the token-by-token recurrence
of Laplace 3B on AWS Trainium2, "GLA mixer"; training differentiates through
the chunked state updates, "Challenge 1"). Tolerances as for the forward:
max relative error (normwise per tensor) 2e-3 for bf16 inputs, 1e-5 for fp32.
"""
import dataclasses
import os

import numpy as np
import pytest

import gpu_util as gu
from gated_linear_attention_amd import synth
from oracle import gla_oracle as orc

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dS0")
W = synth.WORKLOADS


def run_bwd(q, k, v, lg, S0, cu, dO, dS_T, dtype, C):
    import torch
    import gated_linear_attention_amd as gla
    td = gu.in_dtype(dtype)
    res = gla.bwd_chunked(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lg),
                          gu.dev(dO, td), S0=gu.dev(S0), cu_seqlens=gu.dev(cu),
                          dS_T=gu.dev(dS_T), chunk_size=C)
    torch.cuda.synchronize()
    return [gu.host(x) for x in res]


def check_bwd(q, k, v, lg, S0, cu, dO, dS_T, dtype, C=64, heads=None, tight=None):
    got = run_bwd(q, k, v, lg, S0, cu, dO, dS_T, dtype, C)
    if heads is not None:
        got = [g[:, :, heads] if g.ndim >= 3 and g.shape[0] == q.shape[0] and n != "dS0"
               else g[:, heads] for g, n in zip(got, NAMES)]
    ref = orc.recurrent_backward(q, k, v, lg, dO, dS_T, S0, cu, heads=heads)
    tol = gu.TOL_BF16 if dtype == "bf16" else gu.TOL_F32
    errs = [orc.normwise_error(g, r) for g, r in zip(got, ref)]
    gu.say("   " + "  ".join(f"{n} {e:.2e}" for n, e in zip(NAMES, errs)) + f"  (tol {tol:.0e})")
    for n, e in zip(NAMES, errs):
        assert e <= tol, (n, e)
        if tight is not None:
            assert e <= tight, (n, e)


def _inputs(w, seed, B=None, T=None, H=None, lengths=None, final_state=True):
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w, seed=seed, B=B, T=T, H=H, lengths=lengths)
    Bq, Tq, Hq = q.shape[:3]
    N = Bq if cu is None else len(cu) - 1
    dO, dS_T = synth.make_backward_grads(w, Bq, Tq, Hq, N, seed=seed + 7,
                                         final_state=final_state)
    return q, k, v, lg, S0, cu, dO, dS_T


def _shape(dk, dv, s0=0.02):
    return dataclasses.replace(W["train_2k"], dk=dk, dv=dv, s0_std=s0)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [64, 300, 1])
def test_bwd_bf16_shapes(dk, dv, T):
    """Several chunks, a ragged tail, one token; nonzero S0 and dS_T."""
    gu.say(f"bwd bf16 dk={dk} dv={dv} T={T}")
    check_bwd(*_inputs(_shape(dk, dv), 500 + T + dk + dv, B=2, T=T, H=2), "bf16", tight=1e-4)


@pytest.mark.parametrize("C", [64, 128])
def test_bwd_chunk_sizes(C):
    gu.say(f"bwd bf16 C={C}")
    check_bwd(*_inputs(_shape(128, 128), 600, B=2, T=333, H=2), "bf16", C=C, tight=1e-4)


@pytest.mark.parametrize("C", [64, 128])
def test_bwd_f32_tiny_workload(C):
    """The fp32 workload's shape (B=1, H=2, T=256, d=64), with upstream gradients."""
    gu.say(f"bwd fp32 tiny C={C}")
    check_bwd(*_inputs(W["tiny_f32"], 610), "f32", C=C)


def test_bwd_without_S0_and_dS_T():
    gu.say("bwd bf16 no S0, no dS_T")
    check_bwd(*_inputs(_shape(128, 128, s0=0.0), 620, B=2, T=200, H=2, final_state=False), "bf16",
              tight=1e-4)


@pytest.mark.parametrize("C", [64, 128])
def test_bwd_varlen_edges(C):
    """Empty, one-token, sub-chunk, chunk-edge and multi-chunk sequences packed."""
    gu.say(f"bwd varlen edges C={C}")
    w = dataclasses.replace(W["varlen_64"], H=2)
    lengths = [0, 1, 63, 64, 65, 200, 0, 130]
    check_bwd(*_inputs(w, 630, lengths=lengths), "bf16", C=C, tight=1e-4)


def test_bwd_near_reset_and_unit_gates():
    """l = -20 (a near reset; the chunked form needs finite gates, as the
    forward) and l = 0 (no decay) at chosen tokens."""
    gu.say("bwd near-reset / unit gates")
    q, k, v, lg, S0, cu, dO, dS_T = _inputs(_shape(128, 128), 640, B=2, T=200, H=2)
    lg[:, 70] = -20.0
    lg[1, 130:150] = 0.0
    check_bwd(q, k, v, lg, S0, cu, dO, dS_T, "bf16", tight=1e-4)


@pytest.mark.parametrize("seg,sub", [(64, 1), (192, 1), (256, 4)])
def test_bwd_forced_segment_split(seg, sub, monkeypatch):
    """Long sequences split into segments inside the forward runs (state pass,
    in `sub` pieces per segment, combine, output pass) give the same gradients."""
    gu.say(f"bwd forced split seg={seg} pieces={sub}")
    monkeypatch.setenv("GLA_SEG_LEN", str(seg))
    monkeypatch.setenv("GLA_STATE_SUB", str(sub))
    w = dataclasses.replace(W["varlen_64"], H=2)
    check_bwd(*_inputs(w, 650, lengths=[500, 3, 257, 0, 64]), "bf16", tight=1e-4)


def test_bwd_full_train_2k_sampled_heads():
    """B=8, T=2048, H=16, d=128 bf16 (the training shape), heads 0 and 11 checked."""
    gu.say("bwd train_2k full size, heads 0 and 11")
    w = W["train_2k"]
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    dO, dS_T = synth.make_backward_grads(w, w.B, w.T, w.H, w.B, seed=w.seed + 7)
    check_bwd(q, k, v, lg, S0, cu, dO, dS_T, "bf16", heads=[0, 11], tight=1e-4)
