"""Seeded random sweep of the entry points against the fp64 oracle.

Each case draws its whole configuration from its seed and prints it before
running, so that a failure names it: head shape, input dtype, chunk size,
dense or packed batch (with empty and short sequences), batch and sequence
sizes (including zero tokens), gate strength (from near-reset to near-unit
gates), initial state or none, fixed per-head decays, and forced segment
splits with state pieces. The reference is the token-by-token recurrence of
Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), "GLA mixer", in
fp64; tolerances as everywhere: 2e-3 normwise per (sequence, head) pair for
bf16 inputs, 1e-5 for fp32, and on the 96 x 192 heads the log-gate gradient's
bar times how much its two dot products cancel (capped).
Sizes stay small so the oracle answers in well under a second per case.
"""
import dataclasses

import numpy as np
import pytest

import gpu_util as gu
from gated_linear_attention_amd import synth
from oracle import c_oracle
from oracle import epilogue_oracle as eo
from oracle import gla_oracle as orc

pytestmark = pytest.mark.gpu

FWD_DIMS = [(64, 64), (128, 128), (64, 128), (128, 64), (96, 192)]
BWD_DIMS = [(64, 64), (128, 128), (64, 128), (128, 64)]
GATE_BIAS = [-3.0, 0.0, 3.0, 7.0]  # log g = logsigmoid(N(0,1) + bias): about -3 .. -0.001


def _draw_fwd(seed, dims, allow_fixed):
    rng = np.random.default_rng(seed)
    c = dict(seed=seed)
    c["dk"], c["dv"] = dims[int(rng.integers(len(dims)))]
    c["dtype"] = "bf16" if rng.random() < 0.7 else "f32"
    c["C"] = int(rng.choice([64, 128]))
    c["H"] = int(rng.integers(1, 4))
    if rng.random() < 0.4:
        n = int(rng.integers(1, 7))
        c["lengths"] = [int(x) for x in rng.integers(0, 400, size=n)]
        if rng.random() < 0.3:
            c["lengths"][int(rng.integers(n))] = int(rng.integers(1, 3))
        c["B"], c["T"] = None, None
    else:
        c["lengths"] = None
        c["B"] = int(rng.integers(1, 4))
        c["T"] = int(rng.choice([0, 1, int(rng.integers(2, 64)), int(rng.integers(64, 450))]))
    c["gate_bias"] = float(rng.choice(GATE_BIAS))
    c["s0"] = float(rng.choice([0.0, 0.02]))
    c["fixed"] = bool(allow_fixed and rng.random() < 0.25)
    c["split"] = None
    if rng.random() < 0.3:
        c["split"] = (c["C"] * int(rng.integers(1, 4)), int(rng.integers(1, 4)))
    return c


def _inputs(c, final_grads=False):
    w = synth.Workload("sweep", B=c["B"] or 1, T=c["T"] or 0, H=c["H"], dk=c["dk"], dv=c["dv"],
                       dtype=c["dtype"], gate_bias=c["gate_bias"], s0_std=c["s0"], chunk=c["C"],
                       seed=c["seed"], fixed_decay=c.get("fixed", False))
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w, B=c["B"], T=c["T"], H=c["H"],
                                                    lengths=c["lengths"])
    if not final_grads:
        return q, k, v, lg, S0, cu
    Bq, Tq, Hq = q.shape[:3]
    N = Bq if cu is None else len(cu) - 1
    dO, dS_T = synth.make_backward_grads(w, Bq, Tq, Hq, N, seed=c["seed"] + 7,
                                         final_state=c["seed"] % 2 == 0)
    return q, k, v, lg, S0, cu, dO, dS_T


def _set_split(c, monkeypatch):
    if c["split"]:
        monkeypatch.setenv("GLA_SEG_LEN", str(c["split"][0]))
        monkeypatch.setenv("GLA_STATE_SUB", str(c["split"][1]))


@pytest.mark.parametrize("seed", range(7000, 7032))
def test_forward_sweep(seed, monkeypatch):
    import torch
    import gated_linear_attention_amd as gla
    c = _draw_fwd(seed, FWD_DIMS, allow_fixed=True)
    gu.say(f"forward sweep {c}")
    _set_split(c, monkeypatch)
    q, k, v, lg, S0, cu = _inputs(c)
    td = gu.in_dtype(c["dtype"])
    args = (gu.dev(q, td), gu.dev(k, td), gu.dev(v, td))
    if c["fixed"]:
        o, ST = gla.fwd_chunked_fixed_decay(*args, gu.dev(synth.fixed_log_decays(c["H"])),
                                            gu.dev(S0), gu.dev(cu), chunk_size=c["C"])
    else:
        o, ST = gla.fwd_chunked(*args, gu.dev(lg), gu.dev(S0), gu.dev(cu), chunk_size=c["C"])
    torch.cuda.synchronize()
    o, ST = gu.host(o), gu.host(ST)
    o_ref, S_ref, _ = c_oracle.fwd(q, k, v, lg, S0, cu, nthreads=16)
    if q.shape[1] == 0:  # no tokens: S_T is S0 (or zero), bit for bit
        assert o.size == 0 and np.array_equal(ST, S_ref), "empty batch"
        return
    tol = gu.TOL_BF16 if c["dtype"] == "bf16" else gu.TOL_F32
    eo_, eS = gu.tok_error(o, o_ref, cu), gu.state_error(ST, S_ref)
    gu.say(f"   o err {eo_:.2e}  S_T err {eS:.2e}  (tol {tol:.0e})")
    assert eo_ <= tol and eS <= tol, (eo_, eS)


@pytest.mark.parametrize("seed", range(7100, 7112))
def test_backward_sweep(seed, monkeypatch):
    _backward_case(seed, monkeypatch, BWD_DIMS, scaled_dg=False)


@pytest.mark.parametrize("seed", range(7150, 7156))
def test_backward_sweep_laplace(seed, monkeypatch):
    """The same draws on Laplace 3B's 96 x 192 heads."""
    _backward_case(seed, monkeypatch, [(96, 192)], scaled_dg=True)


def _backward_case(seed, monkeypatch, dims, scaled_dg):
    import torch
    import gated_linear_attention_amd as gla
    c = _draw_fwd(seed, dims, allow_fixed=False)
    # the backward oracle is a per-token numpy loop: keep it small
    if c["lengths"] is not None:
        c["lengths"] = [min(x, 200) for x in c["lengths"]]
    else:
        c["B"], c["T"] = min(c["B"], 2), min(c["T"], 200)
    c["H"] = min(c["H"], 2)
    gu.say(f"backward sweep {c}")
    _set_split(c, monkeypatch)
    q, k, v, lg, S0, cu, dO, dS_T = _inputs(c, final_grads=True)
    td = gu.in_dtype(c["dtype"])
    got = gla.bwd_chunked(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lg),
                          gu.dev(dO, td), S0=gu.dev(S0), cu_seqlens=gu.dev(cu),
                          dS_T=gu.dev(dS_T), chunk_size=c["C"])
    torch.cuda.synchronize()
    got = [gu.host(x) for x in got]
    ref = orc.recurrent_backward(q, k, v, lg, dO, dS_T, S0, cu)
    names = ["dq", "dk", "dv", "dlog_g", "dS0"]
    if q.shape[1] == 0:
        for n, g, r in zip(names, got, ref):
            assert g.size == r.size and np.array_equal(g, r), n
        return
    tol = gu.TOL_BF16 if c["dtype"] == "bf16" else gu.TOL_F32
    *errs, dg_pair = gu.grad_errors(got, ref, cu)
    # the 96 x 192 draws hold dlog_g to the bar times its (capped) cancellation
    tol_dg = gu.dg_tolerance(tol, q, k, ref[0], ref[1]) if scaled_dg else tol
    gu.say("   " + "  ".join(f"{n} {e:.2e}" for n, e in zip(names, errs))
           + f"  (dlog_g per pair {dg_pair:.1e}; tol {tol:.0e}, dlog_g {tol_dg:.1e})")
    for n, e in zip(names, errs):
        assert e <= (tol_dg if n == "dlog_g" else tol), (n, e)


@pytest.mark.parametrize("seed", range(7200, 7212))
def test_decode_sweep(seed):
    """One decode step (dense state, or a slot pool with padded lanes), then
    for half the cases the fused decode + mixer epilogue on the same inputs."""
    import torch
    import gated_linear_attention_amd as gla
    rng = np.random.default_rng(seed)
    dk, dv = FWD_DIMS[int(rng.integers(len(FWD_DIMS)))]
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    N = int(rng.choice([1, int(rng.integers(2, 40)), int(rng.integers(40, 700))]))
    H = int(rng.integers(1, 5))
    pooled = rng.random() < 0.5
    fused = rng.random() < 0.5
    out_bf16 = rng.random() < 0.3
    P = N + int(rng.integers(0, 50)) if pooled else N
    slots = None
    if pooled:
        slots = rng.permutation(P)[:N].astype(np.int32)
        pad = rng.random(N) < 0.15
        slots[pad] = -1
    cfg = dict(seed=seed, dk=dk, dv=dv, dtype=dtype, N=N, H=H, P=P, pooled=pooled, fused=fused,
               out_bf16=out_bf16)
    gu.say(f"decode sweep {cfg}")
    S_np = synth.make_decode_state(P, H, dk, dv, seed=seed + 1)
    q, k, v, lg = synth.make_decode_step_inputs(N, H, dk, dv, seed=seed + 2, dtype=dtype)
    td = gu.in_dtype(dtype)
    S = gu.dev(S_np)
    od = torch.bfloat16 if out_bf16 else torch.float32
    valid = list(range(N)) if slots is None else [n for n in range(N) if slots[n] >= 0]
    idx = valid if slots is None else [int(slots[n]) for n in valid]
    o_ref = np.zeros((N, H, dv))
    S_ref = S_np.astype(np.float64).copy()
    if valid:
        o_v, S_v = orc.decode_step(q[valid], k[valid], v[valid], lg[valid], S_ref[idx])
        o_ref[valid] = o_v
        S_ref[idx] = S_v
    ins = (gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lg))
    if fused:
        a, tw, tier = synth.make_epilogue_params(H, dk, dv, seed=seed + 3, n_tiers=2)
        gout = synth.make_epilogue_inputs(N, H, dk, dv, seed=seed + 4, dtype=dtype)[4]
        w = gla.head_rms_weights(gu.dev(tw), gu.dev(tier))
        got = gla.decode_mixer(*ins, S, gu.dev(gout, td), gu.dev(a), w, 1e-6,
                               slots=None if slots is None else gu.dev(slots), out_dtype=od)
        ref = np.zeros((N, H, dv))
        if valid:
            ref[valid] = eo.mixer_epilogue(o_ref[valid], q[valid], k[valid], v[valid],
                                           gout[valid], a, tw, tier, 1e-6)
    elif slots is None:
        got = gla.decode_step(*ins, S, out_dtype=od)
        ref = o_ref
    else:
        got = gla.decode_step_slots(*ins, S, gu.dev(slots), out_dtype=od)
        ref = o_ref
    torch.cuda.synchronize()
    got = gu.host(got)
    if out_bf16:
        ref = synth.round_bf16(ref.astype(np.float32))
    tol = (gu.TOL_BF16_OUT if out_bf16 else 1e-5)
    e = gu.state_error(got, ref)  # per (sequence, head): [N, H, dv]
    eS = gu.state_error(gu.host(S)[idx], S_ref[idx]) if idx else 0.0
    gu.say(f"   out err {e:.2e}  S err {eS:.2e}")
    assert e <= tol and eS <= 1e-6, (e, eS)
    untouched = sorted(set(range(P)) - set(idx))
    assert np.array_equal(gu.host(S)[untouched], S_np[untouched].astype(np.float64))
    pad = [n for n in range(N) if n not in valid]
    assert np.all(got[pad] == 0.0)
