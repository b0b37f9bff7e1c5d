"""Reset gates in the chunked forward and backward: a log-gate of -inf (g = 0)
restarts the state, S_t = k_t^T v_t (Laplace 3B on AWS Trainium2, "GLA
mixer": the gate multiplies the old state, so a zero gate drops it).

The kernels never form a decay product across a reset (the in-chunk scans
restart there), so a reset at a sequence start, in the middle of a chunk, on
a chunk boundary, on the last token, in a run of consecutive tokens or in a
chunk made only of resets gives the oracle's result within the usual bars.
Log-gates at or below -128 ln 2 (g <= 2^-128) are taken as exact resets too;
the oracle's exp() gives 0 or a value below 1e-38 for them, so they are
checked against it the same way. The backward's log-gate gradient is exactly
0 at a reset (the oracle's g_t <A_t, S_{t-1}>), and no gradient crosses one.
"""
import numpy as np
import pytest

import gpu_util as gu
from gated_linear_attention_amd import synth
from oracle import c_oracle
from oracle import gla_oracle as orc

pytestmark = pytest.mark.gpu

NEG_INF = -np.inf


def plant(lg, where, value=NEG_INF):
    """Copy of the log-gates with `value` at the (b, t, h) positions in `where`."""
    lg = lg.copy()
    for b, t, h in where:
        lg[b, t, h] = value
    return lg


def dense_resets(T, C):
    """Reset positions of a dense batch of 2 sequences x 3 heads: sequence 0,
    head 0 at its first token, mid-chunk, on chunk boundaries of every chunk
    size, twice in a row and on its last token; sequence 1, head 1 over a
    whole chunk (or to the end of the sequence); head 2 none (heads are
    independent)."""
    w = [(0, 0, 0), (0, 37, 0), (0, 64, 0), (0, 128, 0), (0, 100, 0), (0, 101, 0),
         (0, T - 1, 0)]
    if T > 256:
        w += [(0, 256, 0)]
    w += [(1, t, 1) for t in range(C, min(2 * C, T))]
    w += [(1, 5, 0)]
    return w


def fwd_gpu(q, k, v, lg, S0, cu, dtype, C, fixed=False, alias=False):
    import torch
    import gated_linear_attention_amd as gla
    td = gu.in_dtype(dtype)
    S0d = gu.dev(S0)
    if fixed:
        o, ST = gla.fwd_chunked_fixed_decay(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td),
                                            gu.dev(lg), S0d, gu.dev(cu), chunk_size=C)
    else:
        o, ST = gla.fwd_chunked(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lg), S0d,
                                gu.dev(cu), chunk_size=C, S_T=S0d if alias else None)
    torch.cuda.synchronize()
    return gu.host(o), gu.host(ST)


def check_fwd(q, k, v, lg, S0, cu, dtype, C, tight=None, alias=False):
    o, ST = fwd_gpu(q, k, v, lg, S0, cu, dtype, C, alias=alias)
    o_ref, S_ref, _ = c_oracle.fwd(q, k, v, lg, S0, cu, nthreads=16)
    eo = gu.tok_error(o, o_ref, cu)
    eS = gu.state_error(ST, S_ref)
    tol = gu.TOL_BF16 if dtype == "bf16" else gu.TOL_F32
    gu.say(f"   o err {eo:.3e}  S_T err {eS:.3e}  (tol {tol:.0e})")
    assert eo <= tol and eS <= tol, (eo, eS)
    if tight is not None:
        assert eo <= tight and eS <= tight, (eo, eS)


@pytest.mark.parametrize("value", [NEG_INF, -200.0, -1e30])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("C", [64, 128, 256])
def test_reset_forward_dense(C, dtype, value):
    gu.say(f"reset fwd dense C={C} {dtype} value={value}")
    T = 300
    w = synth.Workload("r", B=2, T=T, H=3, dk=64, dv=64, dtype=dtype, gate_bias=3.0,
                       s0_std=0.02, chunk=C, seed=71)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    lg = plant(lg, dense_resets(T, C), value)
    check_fwd(q, k, v, lg, S0, cu, dtype, C, tight=2e-5 if dtype == "bf16" else None)


@pytest.mark.parametrize("dk,dv", [(128, 128), (96, 192)])
@pytest.mark.parametrize("C", [64, 128])
def test_reset_forward_head_shapes(dk, dv, C):
    gu.say(f"reset fwd bf16 dk={dk} dv={dv} C={C}")
    T = 260
    w = synth.Workload("r", B=2, T=T, H=3, dk=dk, dv=dv, dtype="bf16", gate_bias=3.0,
                       s0_std=0.02, chunk=C, seed=72)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    check_fwd(q, k, v, plant(lg, dense_resets(T, C)), S0, cu, "bf16", C, tight=2e-5)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("C", [64, 128])
def test_reset_forward_varlen(C, dtype):
    """Packed sequences with resets on their first and last tokens and inside;
    a reset on a sequence's first token only drops S0."""
    gu.say(f"reset fwd varlen C={C} {dtype}")
    lengths = [0, 1, 63, 64, 65, 200, 130, 7]
    w = synth.Workload("r", B=1, T=0, H=2, dk=128, dv=128, dtype=dtype, gate_bias=3.0,
                       s0_std=0.03, chunk=C, seed=73)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w, lengths=lengths)
    where = []
    for n in range(len(lengths)):
        s, e = int(cu[n]), int(cu[n + 1])
        if e > s:
            where += [(0, s, 0), (0, e - 1, 1), (0, (s + e) // 2, 0)]
    check_fwd(q, k, v, plant(lg, where), S0, cu, dtype, C,
              tight=2e-5 if dtype == "bf16" else None)


@pytest.mark.parametrize("seg,sub,C", [(128, 1, 64), (256, 2, 64), (256, 1, 128)])
@pytest.mark.parametrize("varlen", [False, True])
def test_reset_forward_split(seg, sub, C, varlen, monkeypatch):
    """Segment splits: a reset inside a state-pass piece makes its total
    log-decay -inf, so the combine drops the state before it; resets on
    segment and piece boundaries; S_T written over S0."""
    gu.say(f"reset fwd split seg={seg} sub={sub} C={C} varlen={varlen}")
    monkeypatch.setenv("GLA_SEG_LEN", str(seg))
    monkeypatch.setenv("GLA_STATE_SUB", str(sub))
    w = synth.Workload("r", B=2, T=700, H=2, dk=128, dv=128, dtype="bf16", gate_bias=3.0,
                       s0_std=0.03, chunk=C, seed=74)
    lengths = [700, 0, 37, 600, 129] if varlen else None
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w, lengths=lengths)
    if varlen:
        where = [(0, 128, 0), (0, 300, 0), (0, 256, 1), (0, 737 + 130, 0), (0, 737 + 599, 1)]
    else:
        where = [(0, 128, 0), (0, 300, 0), (0, 256, 1), (1, 0, 0), (1, 699, 1), (1, 384, 0)]
    check_fwd(q, k, v, plant(lg, where), S0, cu, "bf16", C, tight=2e-5, alias=True)


@pytest.mark.parametrize("C", [64, 128])
def test_reset_fixed_decay_every_token(C):
    """A fixed log-decay of -inf resets at every token: o_t = (q_t . k_t) v_t
    and S_T = k_T^T v_T (closed form), while the other heads decay normally."""
    gu.say(f"reset fixed decay, every token, C={C}")
    H = 3
    w = synth.Workload("r", B=2, T=150, H=H, dk=64, dv=64, dtype="bf16", gate_bias=0.0,
                       s0_std=0.02, chunk=C, seed=75, fixed_decay=True)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    lam = synth.fixed_log_decays(H).copy()
    lam[1] = NEG_INF
    o, ST = fwd_gpu(q, k, v, lam, S0, cu, "bf16", C, fixed=True)
    qf, kf, vf = (x.astype(np.float64) for x in (q, k, v))
    o1 = (qf[:, :, 1] * kf[:, :, 1]).sum(-1)[..., None] * vf[:, :, 1]
    S1 = kf[:, -1, 1][:, :, None] * vf[:, -1, 1][:, None, :]
    e1 = max(orc.normwise_error(o[:, :, 1], o1), orc.normwise_error(ST[:, 1], S1))
    lg_full = np.broadcast_to(lam, lg.shape).astype(np.float32).copy()
    o_ref, S_ref, _ = c_oracle.fwd(q, k, v, lg_full, S0, cu, nthreads=16)
    e_all = max(gu.tok_error(o, o_ref), gu.state_error(ST, S_ref))
    gu.say(f"   reset head vs closed form {e1:.2e}; all heads vs oracle {e_all:.2e}")
    assert e1 <= 2e-5 and e_all <= 2e-5, (e1, e_all)


# ------------------------------------------------------------------ backward
NAMES = ("dq", "dk", "dv", "dg", "dS0")


def check_bwd(q, k, v, lg, S0, cu, dO, dS_T, dtype, C, tight=None):
    import torch
    import gated_linear_attention_amd as gla
    td = gu.in_dtype(dtype)
    res = gla.bwd_chunked(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lg),
                          gu.dev(dO, td), S0=gu.dev(S0), cu_seqlens=gu.dev(cu),
                          dS_T=gu.dev(dS_T), chunk_size=C)
    torch.cuda.synchronize()
    got = [gu.host(x) for x in res]
    ref = orc.recurrent_backward(q, k, v, lg, dO, dS_T, S0, cu)
    tol = gu.TOL_BF16 if dtype == "bf16" else gu.TOL_F32
    cancel = 1.0  # the plain bar for dlog_g too
    *errs, dg_pair = gu.grad_errors(got, ref, cu)
    gu.say("   " + "  ".join(f"{n} {e:.2e}" for n, e in zip(NAMES, errs))
           + f"  (dg per pair {dg_pair:.1e}; tol {tol:.0e})")
    # the gradient of a reset gate is exactly zero
    reset = np.isneginf(lg) | (lg <= -88.72283906)
    assert np.all(got[3][reset] == 0.0)
    for n, e in zip(NAMES, errs):
        scale = cancel if n == "dg" else 1.0
        assert e <= tol * scale, (n, e)
        if tight is not None:
            assert e <= tight * scale, (n, e)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("C", [64, 128])
def test_reset_backward_dense(C, dtype):
    gu.say(f"reset bwd dense C={C} {dtype}")
    T = 300
    w = synth.Workload("r", B=2, T=T, H=3, dk=64, dv=64, dtype=dtype, gate_bias=3.0,
                       s0_std=0.02, chunk=C, seed=76)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    dO, dS_T = synth.make_backward_grads(w, 2, T, 3, 2, seed=77)
    check_bwd(q, k, v, plant(lg, dense_resets(T, C)), S0, cu, dO, dS_T, dtype, C,
              tight=1e-4 if dtype == "bf16" else None)


@pytest.mark.parametrize("dk,dv", [(128, 128), (96, 192)])
def test_reset_backward_head_shapes(dk, dv):
    gu.say(f"reset bwd bf16 dk={dk} dv={dv}")
    T = 200
    w = synth.Workload("r", B=2, T=T, H=2, dk=dk, dv=dv, dtype="bf16", gate_bias=3.0,
                       s0_std=0.02, chunk=64, seed=78)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    dO, dS_T = synth.make_backward_grads(w, 2, T, 2, 2, seed=79)
    where = [(0, 0, 0), (0, 37, 0), (0, 64, 1), (0, 199, 0), (1, 100, 1), (1, 101, 1)]
    check_bwd(q, k, v, plant(lg, where), S0, cu, dO, dS_T, "bf16", 64, tight=1e-4)


@pytest.mark.parametrize("C", [64, 128])
def test_reset_backward_varlen_split(C, monkeypatch):
    """Packed batch, forced segment splits, resets on sequence starts and ends
    and on a segment boundary."""
    gu.say(f"reset bwd varlen split C={C}")
    monkeypatch.setenv("GLA_SEG_LEN", "128")
    lengths = [300, 0, 1, 64, 200]
    w = synth.Workload("r", B=1, T=0, H=2, dk=64, dv=64, dtype="bf16", gate_bias=3.0,
                       s0_std=0.02, chunk=C, seed=80)
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w, lengths=lengths)
    N = len(lengths)
    dO, dS_T = synth.make_backward_grads(w, 1, q.shape[1], 2, N, seed=81)
    where = [(0, 0, 0), (0, 128, 0), (0, 299, 1), (0, 300, 1), (0, 301, 0), (0, 365, 0),
             (0, 400, 1)]
    check_bwd(q, k, v, plant(lg, where), S0, cu, dO, dS_T, "bf16", C, tight=1e-4)
