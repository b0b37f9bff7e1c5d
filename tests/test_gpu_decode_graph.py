"""A multi-layer decode step captured once as a HIP graph and replayed.

Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116), "Inference
optimization": eager decode spent its time dispatching small operators one at
a time, compiling the step removed that, and fixed padded batch widths kept
one compiled shape. Here one decode step over several layers (per layer: the
slot-indexed decode against that layer's state pool, then the mixer
epilogue) is captured once; each replay, with fresh inputs written into the
captured buffers by eager work in between, must equal the same step run
eagerly on copies of the pools, bit for bit (same kernels, same inputs), and
the first layer must match the oracle's decode followed by its epilogue.
"""
import numpy as np
import pytest

import gpu_util as gu
from gated_linear_attention_amd import synth
from oracle import epilogue_oracle as eo
from oracle import gla_oracle as orc

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_and_oracle():
    import torch
    import gated_linear_attention_amd as gla
    gu.say("decode graph: 3 layers, 96x192, padded lane")
    L, P, H, dk, dv = 3, 12, 16, 96, 192
    slots_h = [3, -1, 7, 0, 11]
    N = len(slots_h)
    dev = torch.device("cuda:0")
    slots = gu.dev(np.asarray(slots_h, np.int32))
    pools0 = [synth.make_decode_state(P, H, dk, dv, seed=60 + l) for l in range(L)]
    pools = [gu.dev(p) for p in pools0]
    pools_e = [p.clone() for p in pools]
    params = [synth.make_epilogue_params(H, dk, dv, seed=70 + l) for l in range(L)]
    a = [gu.dev(p[0]) for p in params]
    w = [gla.head_rms_weights(gu.dev(p[1]), gu.dev(p[2])) for p in params]
    bf = torch.bfloat16
    # static input and output buffers of the captured step
    q = [torch.zeros((N, H, dk), dtype=bf, device=dev) for _ in range(L)]
    k = [torch.zeros_like(x) for x in q]
    v = [torch.zeros((N, H, dv), dtype=bf, device=dev) for _ in range(L)]
    gate = [torch.zeros_like(x) for x in v]
    lg = [torch.zeros((N, H), dtype=torch.float32, device=dev) for _ in range(L)]
    o = [torch.empty((N, H, dv), dtype=torch.float32, device=dev) for _ in range(L)]
    z = [torch.empty((N, H, dv), dtype=bf, device=dev) for _ in range(L)]
    o_e = [torch.empty_like(x) for x in o]
    z_e = [torch.empty_like(x) for x in z]

    def step(pl, oo, zz):
        for l in range(L):
            gla.decode_step_slots(q[l], k[l], v[l], lg[l], pl[l], slots, o=oo[l])
            gla.mixer_epilogue(oo[l], q[l], k[l], v[l], gate[l], a[l], w[l], 1e-6, z=zz[l])

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(pools, o, z)
    torch.cuda.synchronize()
    for p, p0 in zip(pools, pools0):  # capture ran nothing
        assert np.array_equal(gu.host(p), p0.astype(np.float64))

    ref = [p.astype(np.float64) for p in pools0]
    for r in range(3):
        host_in = []
        for l in range(L):
            qq, kk, vv, gg = synth.make_decode_step_inputs(N, H, dk, dv, seed=800 + 10 * r + l)
            ga = synth.make_epilogue_inputs(N, H, dk, dv, seed=900 + 10 * r + l)[4]
            q[l].copy_(gu.dev(qq, bf))
            k[l].copy_(gu.dev(kk, bf))
            v[l].copy_(gu.dev(vv, bf))
            lg[l].copy_(gu.dev(gg))
            gate[l].copy_(gu.dev(ga, bf))
            host_in.append((qq, kk, vv, gg, ga))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(pools_e, o_e, z_e)
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(o[l], o_e[l]) and torch.equal(z[l], z_e[l]), (r, l)
            assert torch.equal(pools[l], pools_e[l]), (r, l)
        # layer 0 against the oracle: decode on the gathered states, then the epilogue
        qq, kk, vv, gg, ga = host_in[0]
        valid = [n for n, s in enumerate(slots_h) if 0 <= s < P]
        idx = [slots_h[n] for n in valid]
        o_v, S_v = orc.decode_step(qq[valid], kk[valid], vv[valid], gg[valid], ref[0][idx])
        ref[0][idx] = S_v
        a0, tw0, tier0 = params[0]
        z_ref = eo.mixer_epilogue(o_v, qq[valid], kk[valid], vv[valid], ga[valid], a0, tw0, tier0,
                                  1e-6)
        z_ref = synth.round_bf16(z_ref.astype(np.float32))
        e = orc.normwise_error(gu.host(z[0])[valid], z_ref)
        gu.say(f"   replay {r}: layer-0 z err {e:.2e}")
        assert e <= gu.TOL_BF16_OUT, e
        assert np.all(gu.host(o[0])[[n for n in range(N) if n not in valid]] == 0.0)
    eS = orc.normwise_error(gu.host(pools[0]), ref[0])
    assert eS <= 1e-6, eS


def test_graph_of_fused_decode_mixer_matches_eager():
    """The fused decode + epilogue (one kernel per layer) captured the same way:
    replays with fresh inputs equal eager runs on copies of the pools, bit for bit."""
    import torch
    import gated_linear_attention_amd as gla
    gu.say("decode graph: fused decode + epilogue, 3 layers")
    L, P, H, dk, dv = 3, 10, 16, 96, 192
    slots_h = [4, 9, -1, 0]
    N = len(slots_h)
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    slots = gu.dev(np.asarray(slots_h, np.int32))
    pools = [gu.dev(synth.make_decode_state(P, H, dk, dv, seed=160 + l)) for l in range(L)]
    pools_e = [p.clone() for p in pools]
    params = [synth.make_epilogue_params(H, dk, dv, seed=170 + l) for l in range(L)]
    a = [gu.dev(p[0]) for p in params]
    w = [gla.head_rms_weights(gu.dev(p[1]), gu.dev(p[2])) for p in params]
    q = [torch.zeros((N, H, dk), dtype=bf, device=dev) for _ in range(L)]
    k = [torch.zeros_like(x) for x in q]
    v = [torch.zeros((N, H, dv), dtype=bf, device=dev) for _ in range(L)]
    gate = [torch.zeros_like(x) for x in v]
    lg = [torch.zeros((N, H), dtype=torch.float32, device=dev) for _ in range(L)]
    z = [torch.empty((N, H, dv), dtype=bf, device=dev) for _ in range(L)]
    z_e = [torch.empty_like(x) for x in z]

    def step(pl, zz):
        for l in range(L):
            gla.decode_mixer(q[l], k[l], v[l], lg[l], pl[l], gate[l], a[l], w[l], 1e-6,
                             slots=slots, z=zz[l])

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(pools, z)
    torch.cuda.synchronize()
    for r in range(3):
        for l in range(L):
            qq, kk, vv, gg = synth.make_decode_step_inputs(N, H, dk, dv, seed=1800 + 10 * r + l)
            q[l].copy_(gu.dev(qq, bf))
            k[l].copy_(gu.dev(kk, bf))
            v[l].copy_(gu.dev(vv, bf))
            lg[l].copy_(gu.dev(gg))
            gate[l].copy_(gu.dev(synth.make_epilogue_inputs(N, H, dk, dv, seed=1900 + 10 * r + l)[4], bf))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(pools_e, z_e)
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(z[l], z_e[l]) and torch.equal(pools[l], pools_e[l]), (r, l)
        assert torch.count_nonzero(z[0][2]) == 0  # the padded lane
