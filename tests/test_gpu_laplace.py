"""GPU parity at the Laplace 3B mixer shape and for fixed per-head decays.

Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116): the mixer's heads
have d_k = 96 and d_v = 192 ("GLA mixer"), and each head's decay is fixed at
initialisation on a geometric schedule ("Decay schedule"). The forward at this
shape (gla_fwd_chunked), the fixed-decay forward (gla_fwd_chunked_fixed_decay,
no per-token gate stream) and the decode step are checked against the fp64
oracle; the fixed-decay forward must also equal the per-token forward fed the
broadcast decays bit for bit (both evaluate the same gate values in the same
order).
"""
import numpy as np
import pytest

import gpu_util as gu
from gated_linear_attention_amd import synth
from oracle import c_oracle
from oracle import gla_oracle as orc
from test_gpu_fwd import check, run_gpu

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _wl(T, dtype="bf16", C=64, seed=31, s0=0.02, fixed=False, H=3):
    return synth.Workload("t", B=2, T=T, H=H, dk=96, dv=192, dtype=dtype, gate_bias=3.0,
                          s0_std=s0, chunk=C, seed=seed, fixed_decay=fixed)


def run_fixed(q, k, v, lam, S0, cu, dtype, C, out_dtype=None):
    import torch
    import gated_linear_attention_amd as gla
    td = gu.in_dtype(dtype)
    o, ST = gla.fwd_chunked_fixed_decay(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lam),
                                        gu.dev(S0), gu.dev(cu), chunk_size=C,
                                        out_dtype=out_dtype)
    torch.cuda.synchronize()
    return gu.host(o), gu.host(ST)


# ------------------------------------------------------------ 96 x 192 forward
@pytest.mark.parametrize("T", [64, 300, 1])
@pytest.mark.parametrize("C", [64, 128])
def test_laplace_shape_bf16(T, C):
    """Several tiles, a ragged tail chunk, a single token; nonzero S0."""
    gu.say(f"96x192 bf16 T={T} C={C}")
    check(*synth.make_forward_inputs(_wl(T, C=C)), "bf16", C=C, tight=2e-5)


@pytest.mark.parametrize("C", [64, 128])
def test_laplace_shape_f32(C):
    gu.say(f"96x192 f32 C={C}")
    check(*synth.make_forward_inputs(_wl(333, dtype="f32", C=C, seed=32)), "f32", C=C)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_laplace_shape_varlen_and_split(dtype, monkeypatch):
    """Packed edge lengths, with sequences split into 128-token segments."""
    gu.say(f"96x192 varlen + split {dtype}")
    monkeypatch.setenv("GLA_SEG_LEN", "128")
    w = _wl(0, dtype=dtype, seed=33)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w, lengths=[0, 1, 63, 64, 65, 300, 0, 130])
    check(q, k, v, lg, S0, cu, dtype)


def test_laplace_shape_bf16_output():
    import torch
    gu.say("96x192 bf16 output")
    check(*synth.make_forward_inputs(_wl(200, seed=34)), "bf16", out_dtype=torch.bfloat16,
          tol=gu.TOL_BF16_OUT)


# ------------------------------------------------------------ fixed decay
@pytest.mark.parametrize("dk,dv,dtype,C", [(96, 192, "bf16", 64), (96, 192, "bf16", 128),
                                           (128, 128, "bf16", 64), (128, 128, "bf16", 128),
                                           (64, 64, "bf16", 64), (96, 192, "f32", 64),
                                           (128, 128, "f32", 128)])
def test_fixed_decay_equals_broadcast_gates(dk, dv, dtype, C):
    """Fixed decays (schedule of 16 heads, tails and several chunks) give the
    per-token forward's result bit for bit, and both match the oracle."""
    gu.say(f"fixed decay dk={dk} dv={dv} {dtype} C={C}")
    w = synth.Workload("t", B=2, T=333, H=16, dk=dk, dv=dv, dtype=dtype, gate_bias=0.0,
                       s0_std=0.02, chunk=C, seed=35, fixed_decay=True)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    lam = synth.fixed_log_decays(16)
    assert np.array_equal(lg[1, 100], lam)
    o_f, S_f = run_fixed(q, k, v, lam, S0, cu, dtype, C)
    o_g, S_g = run_gpu(q, k, v, lg, S0, cu, dtype, C)
    assert np.array_equal(o_f, o_g) and np.array_equal(S_f, S_g)
    check(q, k, v, lg, S0, cu, dtype, C=C)


@pytest.mark.parametrize("dk,dv", [(96, 192), (128, 128)])
@pytest.mark.parametrize("C", [64, 128])
def test_fixed_decay_varlen_split(C, dk, dv, monkeypatch):
    """Packed sequences split into segments: the state pass sums the fixed
    decays over each segment's own tokens only (96 x 192 heads on the
    twelve-wavefront state pass, 128 x 128 on the K-and-V-only one)."""
    gu.say(f"fixed decay varlen + split C={C} {dk}x{dv}")
    monkeypatch.setenv("GLA_SEG_LEN", "192" if C == 64 else "256")
    w = synth.Workload("t", B=1, T=0, H=16, dk=dk, dv=dv, dtype="bf16", gate_bias=0.0,
                       s0_std=0.02, chunk=C, seed=36, fixed_decay=True)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w, lengths=[700, 0, 37, 321, 129, 1])
    lam = synth.fixed_log_decays(16)
    o_f, S_f = run_fixed(q, k, v, lam, S0, cu, "bf16", C)
    o_g, S_g = run_gpu(q, k, v, lg, S0, cu, "bf16", C)
    assert np.array_equal(o_f, o_g) and np.array_equal(S_f, S_g)
    check(q, k, v, lg, S0, cu, "bf16", C=C)


def test_fixed_decay_rejects_bad_shapes():
    import torch
    import gated_linear_attention_amd as gla
    q = torch.zeros((1, 8, 4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        gla.fwd_chunked_fixed_decay(q, q, q, torch.zeros((1, 8, 4), device="cuda"))
    with pytest.raises(ValueError):
        gla.fwd_chunked_fixed_decay(q, q, q, torch.zeros(3, device="cuda"))


# ------------------------------------------------------------ full size
def test_laplace_2k_full_size():
    """B=8, H=16, T=2048, 96 x 192, bf16, fixed decays through the fixed-decay
    entry point at both chunk sizes: every (sequence, head) pair, each held to
    its own normwise bar (the heads' magnitudes differ by more than 10x:
    half-lives of 1 to 2,048 tokens)."""
    gu.say("laplace_2k full size")
    w = W["laplace_2k"]
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    o_ref, S_ref, _ = c_oracle.fwd(q, k, v, lg, None, None, nthreads=16)
    for C in (64, 128):
        o, ST = run_fixed(q, k, v, synth.fixed_log_decays(w.H), S0, cu, "bf16", C)
        eo, eS = gu.tok_error(o, o_ref), gu.state_error(ST, S_ref)
        gu.say(f"   C={C}: o err {eo:.3e}  S_T err {eS:.3e}")
        assert eo <= 1e-4 and eS <= 1e-4, (C, eo, eS)


# ------------------------------------------------------------ decode
def test_laplace_decode_chain():
    """256 sequences x 16 heads of 96 x 192 fp32 state, 20 chained steps with
    the fixed decays; every (sequence, head) pair at every step."""
    import torch
    import gated_linear_attention_amd as gla
    gu.say("laplace decode chain")
    N, H, dk, dv = 256, 16, 96, 192
    S_np = synth.make_decode_state(N, H, dk, dv, seed=37)
    S = gu.dev(S_np)
    S_ref = S_np.astype(np.float64)
    lg = np.ascontiguousarray(np.broadcast_to(synth.fixed_log_decays(H), (N, H)))
    worst = 0.0
    for s in range(20):
        q, k, v, _ = synth.make_decode_step_inputs(N, H, dk, dv, seed=5000 + s)
        o = gla.decode_step(gu.dev(q, torch.bfloat16), gu.dev(k, torch.bfloat16),
                            gu.dev(v, torch.bfloat16), gu.dev(lg), S)
        o_ref, _ = c_oracle.decode(q, k, v, lg, S_ref, nthreads=16)
        worst = max(worst, gu.state_error(gu.host(o), o_ref))
    eS = gu.state_error(gu.host(S), S_ref)
    gu.say(f"   o err {worst:.2e}  S err {eS:.2e}")
    assert worst <= 1e-5 and eS <= 1e-6, (worst, eS)
