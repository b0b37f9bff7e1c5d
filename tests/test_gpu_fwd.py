"""GPU parity of the chunked forward (gla_fwd_chunked) against the fp64 oracle.

The oracle is the token-by-token recurrence of Laplace 3B on AWS Trainium2
(automationscribe.com/?p=7116), "GLA mixer"; the kernels compute its chunked
form ("Challenge 1"). Tolerances: max relative error (normwise per tensor)
2e-3 for bf16 inputs with fp32 accumulation, 1e-5 for fp32 inputs.
"""
import os

import numpy as np
import pytest

import gpu_util as gu
from gated_linear_attention_amd import synth
from oracle import c_oracle
from oracle import gla_oracle as orc

pytestmark = pytest.mark.gpu


def run_gpu(q, k, v, lg, S0, cu, dtype, C=64, out_dtype=None, alias=False):
    import torch
    import gated_linear_attention_amd as gla
    td = gu.in_dtype(dtype)
    S0d = gu.dev(S0)
    o, ST = gla.fwd_chunked(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lg), S0d,
                            gu.dev(cu), chunk_size=C, out_dtype=out_dtype,
                            S_T=S0d if alias else None)
    torch.cuda.synchronize()
    return gu.host(o), gu.host(ST)


def check(q, k, v, lg, S0, cu, dtype, C=64, heads=None, tol=None, out_dtype=None, alias=False,
          tight=None):
    """GPU forward against the C oracle: the largest normwise error over
    (sequence, head) pairs, for o and for S_T."""
    o, ST = run_gpu(q, k, v, lg, S0, cu, dtype, C, out_dtype, alias)
    if heads is not None:
        sl = lambda a: None if a is None else np.ascontiguousarray(a[:, :, heads] if a.ndim >= 3 else a)
        o_ref, S_ref, _ = c_oracle.fwd(sl(q), sl(k), sl(v), sl(lg),
                                       None if S0 is None else np.ascontiguousarray(S0[:, heads]),
                                       cu, nthreads=16)
        o, ST = o[:, :, heads], ST[:, heads]
    else:
        o_ref, S_ref, _ = c_oracle.fwd(q, k, v, lg, S0, cu, nthreads=16)
    if out_dtype is not None:
        o_ref = synth.round_bf16(o_ref.astype(np.float32))
    eo, eS = gu.tok_error(o, o_ref, cu), gu.state_error(ST, S_ref)
    tol = tol if tol is not None else (gu.TOL_BF16 if dtype == "bf16" else gu.TOL_F32)
    gu.say(f"   o err {eo:.3e}  S_T err {eS:.3e}  (tol {tol:.1e})")
    assert eo <= tol and eS <= tol, (eo, eS)
    if tight is not None:
        assert eo <= tight and eS <= tight, (eo, eS)
    return eo, eS


def check_full_size(name, tight):
    """A full-size workload at both chunk sizes, in the launch configuration
    the benchmark times, against one oracle run over every sequence and head."""
    w = W[name]
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    o_ref, S_ref, used = c_oracle.fwd(q, k, v, lg, S0, cu, nthreads=16)
    gu.say(f"   oracle: {used} threads")
    for C in (64, 128):
        o, ST = run_gpu(q, k, v, lg, S0, cu, w.dtype, C)
        eo, eS = gu.tok_error(o, o_ref, cu), gu.state_error(ST, S_ref)
        gu.say(f"   C={C}: o err {eo:.3e}  S_T err {eS:.3e} (max over {o_ref.shape[2]} heads "
               f"x {len(S_ref)} sequences)")
        assert eo <= gu.TOL_BF16 and eS <= gu.TOL_BF16, (C, eo, eS)
        assert eo <= tight and eS <= tight, (C, eo, eS)
        del o, ST


W = synth.WORKLOADS


@pytest.mark.parametrize("C", [64, 128, 256])
def test_tiny_f32_workload(C):
    """B=1, H=2, T=256, d=64, fp32 inputs, S0 = 0."""
    gu.say(f"tiny fp32 workload C={C}")
    w = W["tiny_f32"]
    check(*synth.make_forward_inputs(w), "f32", C=C)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [64, 300, 1])
@pytest.mark.parametrize("C", [64, 128, 256])
def test_bf16_shapes(dk, dv, T, C):
    """Several tiles, a ragged tail chunk, a single token; nonzero S0."""
    gu.say(f"bf16 dk={dk} dv={dv} T={T} C={C}")
    w = synth.Workload("t", B=2, T=T, H=3, dk=dk, dv=dv, dtype="bf16", gate_bias=3.0,
                       s0_std=0.02, chunk=C, seed=11)
    check(*synth.make_forward_inputs(w), "bf16", C=C, tight=2e-5)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
@pytest.mark.parametrize("C", [64, 128, 256])
def test_f32_shapes(dk, dv, C):
    gu.say(f"f32 dk={dk} dv={dv} C={C}")
    w = synth.Workload("t", B=2, T=333, H=2, dk=dk, dv=dv, dtype="f32", gate_bias=2.0,
                       s0_std=0.02, chunk=C, seed=12)
    check(*synth.make_forward_inputs(w), "f32", C=C)


def test_bf16_output_dtype():
    import torch
    gu.say("bf16 output")
    w = synth.Workload("t", B=1, T=200, H=2, dk=128, dv=128, dtype="bf16", gate_bias=3.0,
                       s0_std=0.02, chunk=64, seed=13)
    check(*synth.make_forward_inputs(w), "bf16", out_dtype=torch.bfloat16, tol=gu.TOL_BF16_OUT)


def test_state_aliasing_S0_S_T():
    gu.say("S_T aliases S0")
    w = synth.Workload("t", B=2, T=190, H=2, dk=128, dv=128, dtype="bf16", gate_bias=3.0,
                       s0_std=0.05, chunk=64, seed=14)
    check(*synth.make_forward_inputs(w), "bf16", alias=True)


@pytest.mark.parametrize("dtype,C", [("bf16", 64), ("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("varlen", [False, True])
def test_state_aliasing_with_split(dtype, C, varlen, monkeypatch):
    """S_T written over S0 while sequences run as several segments: the first
    segment reads S0 while the last one, another workgroup, writes S_T; the
    first reads a copy of S0 made by the combine."""
    gu.say(f"S_T aliases S0 with a split: {dtype} C={C} varlen={varlen}")
    monkeypatch.setenv("GLA_SEG_LEN", "128" if C == 64 else "256")
    monkeypatch.setenv("GLA_STATE_SUB", "2")
    w = synth.Workload("t", B=2, T=600, H=3, dk=64, dv=64, dtype=dtype, gate_bias=3.0,
                       s0_std=0.05, chunk=C, seed=30)
    lengths = [600, 0, 100, 513] if varlen else None
    check(*synth.make_forward_inputs(w, lengths=lengths), dtype, C=C, alias=True)


@pytest.mark.parametrize("gate", ["zero", "strong"])
def test_gate_extremes(gate):
    """l = 0 (no decay: plain causal linear attention) and l = -20 per token."""
    gu.say(f"gate extreme {gate}")
    w = synth.Workload("t", B=1, T=150, H=2, dk=64, dv=64, dtype="bf16", gate_bias=3.0,
                       s0_std=0.02, chunk=64, seed=15)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    lg = np.zeros_like(lg) if gate == "zero" else np.full_like(lg, -20.0)
    check(q, k, v, lg, S0, cu, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("C", [64, 128])
def test_growing_state(dtype, C):
    """l > 0 (a growing state) is computed as given: l = +0.03 per token over
    150 tokens, about 90x growth, with S0."""
    gu.say(f"growing state {dtype} C={C}")
    w = synth.Workload("t", B=2, T=150, H=2, dk=64, dv=64, dtype=dtype, gate_bias=3.0,
                       s0_std=0.02, chunk=C, seed=29)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    check(q, k, v, np.full_like(lg, 0.03), S0, cu, dtype, C=C)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_with_edge_lengths(dtype):
    """Packed batch with empty, length-1, sub-chunk and multi-chunk sequences."""
    gu.say(f"varlen edge lengths {dtype}")
    w = synth.Workload("t", B=1, T=0, H=3, dk=128, dv=128, dtype=dtype, gate_bias=3.0,
                       s0_std=0.02, chunk=64, seed=16)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w, lengths=[0, 1, 63, 64, 65, 200, 0, 130, 7])
    check(q, k, v, lg, S0, cu, dtype)


@pytest.mark.parametrize("seg,C", [(64, 64), (128, 64), (192, 64), (256, 128)])
@pytest.mark.parametrize("varlen", [False, True])
def test_forced_segment_split(seg, C, varlen, monkeypatch):
    """Sequences split into segments: state pass, combine, output pass."""
    gu.say(f"segment split seg_len={seg} C={C} varlen={varlen}")
    monkeypatch.setenv("GLA_SEG_LEN", str(seg))
    w = synth.Workload("t", B=2, T=500, H=2, dk=128, dv=128, dtype="bf16", gate_bias=3.0,
                       s0_std=0.03, chunk=C, seed=17)
    lengths = [500, 0, 37, 321, 129] if varlen else None
    check(*synth.make_forward_inputs(w, lengths=lengths), "bf16", C=C)


@pytest.mark.parametrize("seg,sub,C", [(256, 4, 64), (320, 3, 64), (384, 2, 128)])
@pytest.mark.parametrize("varlen", [False, True])
def test_forced_state_pieces(seg, sub, C, varlen, monkeypatch):
    """Segments whose states the state pass computes in several pieces, which
    the combine chains (including a shorter last piece: 320 = 3 x 128 - 64)."""
    gu.say(f"state pieces seg_len={seg} n_sub={sub} C={C} varlen={varlen}")
    monkeypatch.setenv("GLA_SEG_LEN", str(seg))
    monkeypatch.setenv("GLA_STATE_SUB", str(sub))
    w = synth.Workload("t", B=2, T=1000, H=2, dk=128, dv=128, dtype="bf16", gate_bias=3.0,
                       s0_std=0.03, chunk=C, seed=27)
    lengths = [1000, 0, 37, 700, 129, 333] if varlen else None
    check(*synth.make_forward_inputs(w, lengths=lengths), "bf16", C=C, tight=2e-5)


@pytest.mark.parametrize("dtype,dk,dv,T", [("bf16", 128, 128, 700), ("bf16", 64, 64, 640),
                                          ("f32", 64, 64, 500)])
@pytest.mark.parametrize("alias", [False, True])
def test_dense_plan_equals_packed_plan(dtype, dk, dv, T, alias, monkeypatch):
    """A dense batch is planned in closed form, a packed one by the counting
    sort: the same sequences with the same segment length and pieces, once
    dense and once as cu_seqlens of equal lengths, give the same outputs and
    final states bit for bit (the item order differs, the arithmetic of an
    item does not)."""
    gu.say(f"dense plan vs packed plan {dtype} {dk}x{dv} T={T} alias={alias}")
    monkeypatch.setenv("GLA_SEG_LEN", "256")
    monkeypatch.setenv("GLA_STATE_SUB", "2")
    w = synth.Workload("t", B=3, T=T, H=2, dk=dk, dv=dv, dtype=dtype, gate_bias=3.0,
                       s0_std=0.03, chunk=64, seed=37)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    assert cu is None
    o_d, S_d = run_gpu(q, k, v, lg, S0, None, dtype, alias=alias)
    B = q.shape[0]
    flat = lambda x: x.reshape((1, B * T) + x.shape[2:])
    cu_p = (np.arange(B + 1) * T).astype(np.int32)
    o_p, S_p = run_gpu(flat(q), flat(k), flat(v), flat(lg), S0, cu_p, dtype, alias=alias)
    np.testing.assert_array_equal(o_d.reshape(o_p.shape), o_p)
    np.testing.assert_array_equal(S_d, S_p)
    check(q, k, v, lg, S0, None, dtype, tight=2e-5 if dtype == "bf16" else None)


def test_forced_state_pieces_f32(monkeypatch):
    gu.say("state pieces fp32")
    monkeypatch.setenv("GLA_SEG_LEN", "256")
    monkeypatch.setenv("GLA_STATE_SUB", "4")
    w = synth.Workload("t", B=1, T=900, H=2, dk=64, dv=64, dtype="f32", gate_bias=3.0,
                       s0_std=0.03, chunk=64, seed=28)
    check(*synth.make_forward_inputs(w), "f32")


def test_forced_segment_split_f32(monkeypatch):
    gu.say("segment split fp32")
    monkeypatch.setenv("GLA_SEG_LEN", "128")
    w = synth.Workload("t", B=1, T=450, H=2, dk=64, dv=64, dtype="f32", gate_bias=3.0,
                       s0_std=0.03, chunk=64, seed=18)
    check(*synth.make_forward_inputs(w), "f32")


def test_chunk_size_independence_f32():
    import torch
    gu.say("C=64 vs C=128 (fp32)")
    w = synth.Workload("t", B=1, T=400, H=2, dk=64, dv=64, dtype="f32", gate_bias=3.0,
                       s0_std=0.02, chunk=64, seed=19)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    o1, S1 = run_gpu(q, k, v, lg, S0, cu, "f32", C=64)
    o2, S2 = run_gpu(q, k, v, lg, S0, cu, "f32", C=128)
    assert orc.normwise_error(o1, o2) <= 1e-5 and orc.normwise_error(S1, S2) <= 1e-5


# ----------------------------------------------------------- full-size workloads
def test_train_2k_full_size():
    """B=8, H=16, T=2048, d=128, bf16, S0 = 0: every head of every sequence."""
    gu.say("train_2k full size")
    check_full_size("train_2k", tight=1e-4)


def test_prefill_64k_full_size():
    """B=1, H=32, T=65536, d=128, bf16, nonzero S0, split into segments: all 32
    heads over the whole sequence."""
    gu.say("prefill_64k full size")
    check_full_size("prefill_64k", tight=1e-4)


def test_varlen_64_full_size():
    """64 packed sequences, lengths uniform in [128, 8192], H=16, d=128, bf16:
    every (sequence, head) pair."""
    gu.say("varlen_64 full size")
    check_full_size("varlen_64", tight=1e-4)


def test_binding_refuses_misaligned_views():
    """A contiguous view that starts 4 bytes into its storage is refused by the
    binding (before any launch) with a message; its copy runs."""
    import torch
    import gated_linear_attention_amd as gla
    gu.say("misaligned views refused")
    dev = torch.device("cuda:0")
    n = 64 * 64
    buf = torch.randn(n + 8, device=dev).to(torch.bfloat16)
    q = buf[2:2 + n].view(1, 64, 1, 64)  # 4 bytes past a 16-byte boundary
    assert q.is_contiguous() and q.data_ptr() % 16 == 4
    k = torch.randn((1, 64, 1, 64), device=dev).to(torch.bfloat16)
    g = torch.full((1, 64, 1), -0.1, device=dev)
    with pytest.raises(ValueError, match="16-byte boundary"):
        gla.fwd_chunked(q, k, k, g)
    o, _ = gla.fwd_chunked(q.clone(), k, k, g)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
