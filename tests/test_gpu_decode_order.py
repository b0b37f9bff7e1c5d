"""GPU checks of the decode steps' streaming order.

The serving engine's batch names one pool slot per request (Laplace 3B on AWS
Trainium2, "Inference optimization"); gla_decode_slot_order lists the
requests by slot so that the states stream through HBM in address order, and
the dense step streams its requests in groups. The order changes which
workgroup serves which request, never the arithmetic of a request, so:

* gla_decode_slot_order returns a permutation of 0 .. N-1 that lists the
  valid slots in the pool's streaming order (unique for distinct slots) and
  the padded lanes last, and beside it each position's slot. The streaming
  order, as the header states it: where an entry's size divides 4 MiB and
  the pool holds three or more whole 4 MiB blocks, the blocks in the
  sequence 0, s, 2s, ... (mod the block count; s the first of 3, 5, 7, ...
  coprime with it), slots ascending within a block, then the entries past
  the last whole block ascending; otherwise slots ascending. The test walks
  that block sequence itself (no modular inverse);
* a step with the order gives bit for bit the outputs and pool of the same
  step without it (slot decode and the fused decode + epilogue);
* the dense step at batch sizes that leave a tail after the last whole group,
  or whose group count shares a factor with the first strides, still serves
  every request exactly once (every pair checked against the fp64 oracle).
"""
import math

import numpy as np
import pytest

import gpu_util as gu
from gated_linear_attention_amd import synth
from oracle import gla_oracle as orc

pytestmark = pytest.mark.gpu


def _order(slots, P, slot_bytes=0):
    import gated_linear_attention_amd as gla
    return gu.host(gla.slot_order(gu.dev(np.asarray(slots, np.int32)), P, slot_bytes)).astype(
        np.int64)


def _pool_rank(P, slot_bytes):
    """Rank of every pool entry in the streaming order: the blocks' visiting
    sequence 0, s, 2s, ... walked step by step."""
    rank = np.arange(P, dtype=np.int64)
    group = 4 << 20
    if slot_bytes <= 0 or slot_bytes > group or group % slot_bytes:
        return rank
    gs = group // slot_bytes
    nb = P // gs
    strides = [a for a in (3, 5, 7, 11, 13, 17, 19, 23) if math.gcd(a, nb) == 1]
    if nb < 3 or not strides:
        return rank
    s = strides[0]
    b, seen = 0, set()
    for j in range(nb):  # j-th block visited: j * s mod nb
        assert b not in seen
        seen.add(b)
        rank[b * gs:(b + 1) * gs] = j * gs + np.arange(gs)
        b = (b + s) % nb
    return rank


def _check_order(slots, P, order2, slot_bytes=0):
    """order2 [2, N]: a permutation of the requests (valid slots in the
    pool's streaming order, padded lanes last), then each position's slot."""
    slots = np.asarray(slots, np.int64)
    N = len(slots)
    assert order2.shape == (2, N)
    order = order2[0]
    assert sorted(order.tolist()) == list(range(N)), "not a permutation"
    np.testing.assert_array_equal(order2[1], slots[order])
    valid = (slots >= 0) & (slots < P)
    nv = int(valid.sum())
    head = order[:nv]
    assert np.all(valid[head]) and not np.any(valid[order[nv:]])  # padded lanes last
    rank = _pool_rank(P, slot_bytes)
    assert np.all(np.diff(rank[slots[head]]) >= 0)               # streaming order


@pytest.mark.parametrize("slot_bytes", [0, 1 << 20])
@pytest.mark.parametrize("N,P,pad", [(1, 1, 0), (5, 8, 2), (1280, 2048, 0), (1280, 2048, 37),
                                     (5000, 32768, 11), (3000, 3000, 0), (700, 256, 0)])
def test_slot_order_lists_requests_in_pool_order(N, P, pad, slot_bytes):
    gu.say(f"slot order N={N} P={P} padded={pad} entry {slot_bytes} B")
    rng = np.random.default_rng(N + P)
    if N <= P:
        slots = rng.permutation(P)[:N]
    else:  # more requests than slots: duplicates (ordered arbitrarily among themselves)
        slots = rng.integers(0, P, size=N)
    slots = slots.astype(np.int64)
    if pad:
        lanes = rng.choice(N, size=pad, replace=False)
        slots[lanes[: pad // 2]] = -1
        slots[lanes[pad // 2:]] = P + rng.integers(0, 5, size=pad - pad // 2)
    order = _order(slots, P, slot_bytes)
    _check_order(slots, P, order, slot_bytes)
    if N <= P and not pad:  # distinct slots: the order is unique
        rank = _pool_rank(P, slot_bytes)
        np.testing.assert_array_equal(order[0], np.argsort(rank[slots], kind="stable"))


@pytest.mark.parametrize("P,slot_bytes,blocks", [
    (2050, 1 << 20, 512),     # 512 blocks of four, stride 3, a tail of two entries
    (60, 1 << 20, 15),        # 15 blocks: 3 and 5 share a factor with it, stride 7
    (32768, 64 << 10, 512),   # 64 KiB entries, blocks of 64
    (400, 32 << 10, 3),       # three blocks of 128 (the fewest that are strided), tail 16
    (8, 1 << 20, 0),          # two whole blocks: slot order
    (3000, 3 << 20, 0),       # 3 MiB entries do not tile 4 MiB: slot order
    (3000, 8 << 20, 0),       # larger than a block: slot order
    (3000, (1 << 20) + 4, 0)])
def test_slot_order_block_cases(P, slot_bytes, blocks):
    """Every slot of the pool requested once, in a random batch order: the
    order is the streaming order itself."""
    gu.say(f"slot order over a whole pool P={P}, entry {slot_bytes} B, {blocks} blocks")
    slots = np.random.default_rng(P).permutation(P).astype(np.int64)
    order = _order(slots, P, slot_bytes)
    _check_order(slots, P, order, slot_bytes)
    rank = _pool_rank(P, slot_bytes)
    if blocks == 0:
        np.testing.assert_array_equal(rank, np.arange(P))
    np.testing.assert_array_equal(np.sort(rank), np.arange(P))
    np.testing.assert_array_equal(rank[order[1]], np.arange(P))


def test_slot_order_all_padded_and_empty():
    gu.say("slot order: all padded, and N = 0")
    import torch
    import gated_linear_attention_amd as gla
    order = _order([-1, 9, -3, 4], 4)
    _check_order([-1, 9, -3, 4], 4, order)
    assert tuple(gla.slot_order(torch.empty((0,), dtype=torch.int32, device="cuda"), 8).shape) \
        == (2, 0)


def _slot_step(N, P, H, dk, dv, slots, order, steps=2, seed=0):
    import gated_linear_attention_amd as gla
    pool = gu.dev(synth.make_decode_state(P, H, dk, dv, seed=40 + seed))
    sl = gu.dev(np.asarray(slots, np.int32))
    outs = []
    for step in range(steps):
        q, k, v, lg = synth.make_decode_step_inputs(N, H, dk, dv, seed=900 + 10 * seed + step)
        td = gu.in_dtype("bf16")
        o = gla.decode_step_slots(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lg), pool,
                                  sl, order=order)
        outs.append(gu.host(o))
    return outs, gu.host(pool)


@pytest.mark.parametrize("N,P,H,dk,dv", [(1280, 2048, 2, 128, 128), (300, 512, 4, 96, 192),
                                         (40, 64, 2, 128, 128), (333, 400, 2, 64, 64)])
def test_slot_decode_with_order_is_bit_identical(N, P, H, dk, dv):
    import gated_linear_attention_amd as gla
    gu.say(f"slot decode with and without order N={N} P={P} H={H} {dk}x{dv}")
    rng = np.random.default_rng(N)
    slots = rng.permutation(P)[:N].astype(np.int64)
    slots[::17] = -1
    order = gla.slot_order(gu.dev(slots.astype(np.int32)), P, H * dk * dv * 4)
    _check_order(slots, P, gu.host(order).astype(np.int64), H * dk * dv * 4)
    o_a, pool_a = _slot_step(N, P, H, dk, dv, slots, None)
    o_b, pool_b = _slot_step(N, P, H, dk, dv, slots, order)
    for a, b in zip(o_a, o_b):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(pool_a, pool_b)


@pytest.mark.parametrize("dk,dv", [(128, 128), (96, 192)])
def test_decode_mixer_with_order_is_bit_identical(dk, dv):
    import gated_linear_attention_amd as gla
    gu.say(f"decode + epilogue with and without order {dk}x{dv}")
    N, P, H = 600, 1000, 2
    rng = np.random.default_rng(5)
    slots = rng.permutation(P)[:N].astype(np.int64)
    slots[3::50] = -1
    sl = gu.dev(slots.astype(np.int32))
    order = gla.slot_order(sl, P, H * dk * dv * 4)
    _check_order(slots, P, gu.host(order).astype(np.int64), H * dk * dv * 4)
    a, tw, tier = synth.make_epilogue_params(H, dk, dv, seed=3, n_tiers=2)
    w = gla.head_rms_weights(gu.dev(tw), gu.dev(tier))
    q, k, v, lg = synth.make_decode_step_inputs(N, H, dk, dv, seed=77)
    gout = synth.make_epilogue_inputs(N, H, dk, dv, seed=78)[4]
    td = gu.in_dtype("bf16")
    res = []
    for ordr in (None, order):
        pool = gu.dev(synth.make_decode_state(P, H, dk, dv, seed=4))
        z = gla.decode_mixer(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lg), pool,
                             gu.dev(gout, td), gu.dev(a), w, 1e-6, slots=sl, order=ordr)
        res.append((gu.host(z), gu.host(pool)))
    np.testing.assert_array_equal(res[0][0], res[1][0])
    np.testing.assert_array_equal(res[0][1], res[1][1])


@pytest.mark.parametrize("N,H,dk,dv", [(1203, 1, 128, 128), (1290, 1, 128, 128),
                                       (300, 1, 128, 128), (260, 2, 96, 192),
                                       (1027, 1, 64, 64)])
def test_dense_decode_group_order_serves_every_request(N, H, dk, dv):
    """Requests are grouped by 4 MiB of state: 1,203 heads of 64 KiB are 18
    groups of 64 (a multiple of three: stride five) and a tail of 51; 1,290
    are 20 groups and 10; 300 run on the column-sliced kernel (4 groups and
    44); 1,027 heads of 64 x 64 are 4 groups of 256 and 3; 96 x 192 heads do
    not tile 4 MiB and run in launch order. Every (request, head) pair
    against the oracle, two chained steps."""
    import gated_linear_attention_amd as gla
    gu.say(f"dense decode order N={N} H={H} {dk}x{dv}")
    S_np = synth.make_decode_state(N, H, dk, dv, seed=12)
    ref = S_np.astype(np.float64)
    S = gu.dev(S_np)
    td = gu.in_dtype("bf16")
    for step in range(2):
        q, k, v, lg = synth.make_decode_step_inputs(N, H, dk, dv, seed=300 + step)
        o = gu.host(gla.decode_step(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lg), S))
        o_ref, ref = orc.decode_step(q, k, v, lg, ref)
        eo = max(orc.normwise_error(o[n, h], o_ref[n, h]) for n in range(N) for h in range(H))
        assert eo <= 1e-5, (step, eo)
    S_gpu = gu.host(S)
    eS = max(orc.normwise_error(S_gpu[n, h], ref[n, h]) for n in range(N) for h in range(H))
    gu.say(f"   o err {eo:.2e}  S err {eS:.2e}")
    assert eS <= 1e-6


def test_dense_decode_mixer_group_order_serves_every_request():
    """The fused decode + epilogue on a dense batch grouped by 4 MiB (four
    64 KiB heads a request: 12 groups of 16, stride five, and a tail of 8)."""
    import gated_linear_attention_amd as gla
    from oracle import epilogue_oracle as eo
    N, H, dk, dv = 200, 4, 128, 128
    gu.say("dense decode + epilogue, grouped order")
    S_np = synth.make_decode_state(N, H, dk, dv, seed=21)
    S = gu.dev(S_np)
    a, tw, tier = synth.make_epilogue_params(H, dk, dv, seed=22, n_tiers=2)
    w = gla.head_rms_weights(gu.dev(tw), gu.dev(tier))
    q, k, v, lg = synth.make_decode_step_inputs(N, H, dk, dv, seed=23)
    gout = synth.make_epilogue_inputs(N, H, dk, dv, seed=24)[4]
    td = gu.in_dtype("bf16")
    z = gu.host(gla.decode_mixer(gu.dev(q, td), gu.dev(k, td), gu.dev(v, td), gu.dev(lg), S,
                                 gu.dev(gout, td), gu.dev(a), w, 1e-6))
    o_ref, S_ref = orc.decode_step(q, k, v, lg, S_np.astype(np.float64))
    z_ref = eo.mixer_epilogue(o_ref, q, k, v, gout, a, tw, tier, 1e-6)
    ez = max(orc.normwise_error(z[n, h], z_ref[n, h]) for n in range(N) for h in range(H))
    S_gpu = gu.host(S)
    eS = max(orc.normwise_error(S_gpu[n, h], S_ref[n, h]) for n in range(N) for h in range(H))
    gu.say(f"   z err {ez:.2e}  S err {eS:.2e}")
    assert ez <= 1e-5 and eS <= 1e-6
