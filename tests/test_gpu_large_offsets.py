"""Tensors past 2^31 elements: no 32-bit offset anywhere on the path.

A chunked forward and a backward whose inputs each hold more than 2^31
elements (B=1, T=1,049,576, H=32, d=64; an fp32 output is 8.6 GB) and a decode
step whose state holds 4.3e9 fp32 elements (17 GB) at its highest addresses,
and the mixer epilogue over 2.15e9-element rows. The forward's
last head is compared bit for bit with the same head run alone (small tensors,
the same segment plan forced by GLA_SEG_LEN / GLA_STATE_SUB, so the same
arithmetic), and with the fp64 oracle on its last tokens and final state; the
decode step's highest-addressed pairs with the oracle's step. Inputs are drawn
on the device from a seeded torch generator (N(0,1) q, v; k / sqrt(d); gates
logsigmoid(N(0,1) + 3)), since host draws of this size take longer than the run.
The recurrence is that of Laplace 3B on AWS Trainium2
(automationscribe.com/?p=7116), "GLA mixer".
"""
import numpy as np
import pytest

import gpu_util as gu
from oracle import c_oracle
from oracle import gla_oracle as orc

pytestmark = pytest.mark.gpu


def _draw(gen, shape, scale=1.0, dtype=None):
    import torch
    x = torch.randn(shape, generator=gen, device="cuda")
    if scale != 1.0:
        x *= scale
    return x if dtype is None else x.to(dtype)


def test_forward_beyond_2g_elements(monkeypatch):
    import torch
    import gated_linear_attention_amd as gla
    B, T, H, d = 1, (1 << 20) + 1000, 32, 64
    assert B * T * H * d > (1 << 31)
    gu.say(f"large forward: B={B} T={T} H={H} d={d} bf16 ({B * T * H * d / 2**31:.3f} x 2^31 elements per input)")
    monkeypatch.setenv("GLA_SEG_LEN", "65536")
    monkeypatch.setenv("GLA_STATE_SUB", "4")
    gen = torch.Generator(device="cuda").manual_seed(4242)
    bf = torch.bfloat16
    q = _draw(gen, (B, T, H, d), dtype=bf)
    k = _draw(gen, (B, T, H, d), d ** -0.5, bf)
    v = _draw(gen, (B, T, H, d), dtype=bf)
    g = torch.nn.functional.logsigmoid(_draw(gen, (B, T, H)) + 3.0)
    o, S_T = gla.fwd_chunked(q, k, v, g, chunk_size=64)
    torch.cuda.synchronize()
    gu.say("   full batch done")
    hh = H - 1  # the head at the highest addresses
    one = lambda x: x[:, :, hh:hh + 1].contiguous()
    q1, k1, v1, g1 = one(q), one(k), one(v), one(g)
    o_last = o[:, :, hh].clone()
    S_last = S_T[:, hh].clone()
    del o, S_T, q, k, v, g
    torch.cuda.empty_cache()
    o1, S1 = gla.fwd_chunked(q1, k1, v1, g1, chunk_size=64)
    torch.cuda.synchronize()
    assert torch.equal(o_last, o1[:, :, 0]) and torch.equal(S_last, S1[:, 0]), "head alone differs"
    gu.say("   last head bit-identical to the head run alone")
    # the oracle over the whole sequence of that head (fp64, one thread)
    host = lambda x: x.float().cpu().numpy()
    o_ref, S_ref, _ = c_oracle.fwd(host(q1), host(k1), host(v1), host(g1), None, None, nthreads=1)
    tail = 4096
    eo = orc.normwise_error(gu.host(o1[:, -tail:]), o_ref[:, -tail:])
    eS = orc.normwise_error(gu.host(S1), S_ref)
    gu.say(f"   oracle: last {tail} tokens o err {eo:.2e}, S_T err {eS:.2e}")
    assert eo <= gu.TOL_BF16 and eS <= gu.TOL_BF16, (eo, eS)
    del q1, k1, v1, g1, o1, S1, o_last, S_last
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pooled", [False, True])
def test_decode_beyond_4g_state_elements(pooled):
    import torch
    import gated_linear_attention_amd as gla
    H, d = 16, 128
    P = 16400  # state entries; 16400 * 16 * 128 * 128 = 4.3e9 fp32 elements (17.2 GB)
    N = P if not pooled else 40
    gu.say(f"large decode: pool {P} x {H} heads, d={d}, {N} requests, pooled={pooled}")
    gen = torch.Generator(device="cuda").manual_seed(4343)
    S = _draw(gen, (P, H, d, d), 0.02)
    q = _draw(gen, (N, H, d), dtype=torch.bfloat16)
    k = _draw(gen, (N, H, d), d ** -0.5, torch.bfloat16)
    v = _draw(gen, (N, H, d), dtype=torch.bfloat16)
    g = torch.nn.functional.logsigmoid(_draw(gen, (N, H)) + 3.0)
    # sample: the last requests (dense) or requests pointed at the last entries (pooled)
    if pooled:
        slots_h = np.arange(P - N, P, dtype=np.int32)[::-1].copy()
        slots = torch.from_numpy(slots_h).cuda()
        picks = [(n, int(slots_h[n])) for n in (0, 1, N - 1)]
    else:
        picks = [(n, n) for n in (0, N // 2, N - 2, N - 1)]
    S_before = {e: gu.host(S[e]) for _, e in picks}
    if pooled:
        o = gla.decode_step_slots(q, k, v, g, S, slots)
    else:
        o = gla.decode_step(q, k, v, g, S)
    torch.cuda.synchronize()
    host = lambda x: x.float().cpu().numpy()
    for n, e in picks:
        o_ref, S_ref = orc.decode_step(host(q[n:n + 1]), host(k[n:n + 1]), host(v[n:n + 1]),
                                       host(g[n:n + 1]), S_before[e][None])
        eo = orc.normwise_error(gu.host(o[n:n + 1]), o_ref)
        eS = orc.normwise_error(gu.host(S[e:e + 1]), S_ref)
        gu.say(f"   request {n} (entry {e}): o err {eo:.2e}, S err {eS:.2e}")
        assert eo <= 1e-5 and eS <= 1e-6, (n, eo, eS)
    del S, q, k, v, g, o
    torch.cuda.empty_cache()


def test_backward_beyond_2g_elements(monkeypatch):
    """The backward (three forward runs, two reversed, the fused gate dots,
    the gate kernels) at 2.15e9 elements per input: the highest-addressed
    head equals the same head's backward run alone, bit for bit, under the
    same forced segment plan (the head-alone path is checked against the
    oracle by the backward tests at small sizes)."""
    import torch
    import gated_linear_attention_amd as gla
    B, T, H, d = 1, (1 << 20) + 1000, 32, 64
    gu.say(f"large backward: B={B} T={T} H={H} d={d} bf16")
    monkeypatch.setenv("GLA_SEG_LEN", "65536")
    monkeypatch.setenv("GLA_STATE_SUB", "4")
    gen = torch.Generator(device="cuda").manual_seed(4444)
    bf = torch.bfloat16
    q = _draw(gen, (B, T, H, d), dtype=bf)
    k = _draw(gen, (B, T, H, d), d ** -0.5, bf)
    v = _draw(gen, (B, T, H, d), dtype=bf)
    dO = _draw(gen, (B, T, H, d), dtype=bf)
    g = torch.nn.functional.logsigmoid(_draw(gen, (B, T, H)) + 3.0)
    S0 = _draw(gen, (B, H, d, d), 0.02)
    dS_T = _draw(gen, (B, H, d, d), 0.02)
    got = gla.bwd_chunked(q, k, v, g, dO, S0=S0, dS_T=dS_T)
    torch.cuda.synchronize()
    gu.say("   full batch done")
    hh = H - 1
    last = [x[:, :, hh].clone() if x.dim() >= 3 and x.shape[1] == T else x[:, hh].clone()
            for x in got]
    one = lambda x: x[:, :, hh:hh + 1].contiguous()
    ins = (one(q), one(k), one(v), one(g), one(dO))
    S01, dST1 = S0[:, hh:hh + 1].contiguous(), dS_T[:, hh:hh + 1].contiguous()
    del got, q, k, v, dO, g
    torch.cuda.empty_cache()
    alone = gla.bwd_chunked(*ins, S0=S01, dS_T=dST1)
    torch.cuda.synchronize()
    for name, a, b in zip(["dq", "dk", "dv", "dlog_g", "dS0"], last, alone):
        b = b[:, :, 0] if b.dim() >= 3 and b.shape[1] == T else b[:, 0]
        assert torch.equal(a, b), name
    gu.say("   last head bit-identical to the head run alone (dq, dk, dv, dlog_g, dS0)")
    del last, alone, ins
    torch.cuda.empty_cache()


def test_epilogue_beyond_2g_elements():
    """The mixer epilogue over 11.2M rows of 192 channels (2.15e9 elements in
    o, v, g and z): the last rows against the fp64 epilogue oracle."""
    import torch
    import gated_linear_attention_amd as gla
    from gated_linear_attention_amd import synth
    from oracle import epilogue_oracle as eo
    n_tok, H, dk, dv = 700_000, 16, 96, 192
    assert n_tok * H * dv > (1 << 31)
    gu.say(f"large epilogue: {n_tok} tokens x {H} heads, {dk}x{dv}")
    gen = torch.Generator(device="cuda").manual_seed(4545)
    bf = torch.bfloat16
    o = _draw(gen, (n_tok, H, dv))
    q = _draw(gen, (n_tok, H, dk), dtype=bf)
    k = _draw(gen, (n_tok, H, dk), dk ** -0.5, bf)
    v = _draw(gen, (n_tok, H, dv), dtype=bf)
    gt = _draw(gen, (n_tok, H, dv), dtype=bf)
    a, tw, tier = synth.make_epilogue_params(H, dk, dv, seed=46)
    w = gla.head_rms_weights(gu.dev(tw), gu.dev(tier))
    z = gla.mixer_epilogue(o, q, k, v, gt, gu.dev(a), w, 1e-6, out_dtype=torch.float32)
    torch.cuda.synchronize()
    tail = slice(n_tok - 3, n_tok)
    host = lambda x: x[tail].float().cpu().numpy()
    ref = eo.mixer_epilogue(host(o), host(q), host(k), host(v), host(gt), a, tw, tier, 1e-6)
    e = orc.normwise_error(gu.host(z[tail]), ref)
    gu.say(f"   last 3 tokens (48 rows) err {e:.2e}")
    assert e <= 1e-5, e
    del o, q, k, v, gt, z
    torch.cuda.empty_cache()
