"""Pins of the fp64 oracle against closed forms, brute force and invariants.

The oracle (oracle/gla_oracle.py, oracle/gla_oracle.c) implements the GLA
recurrence of Laplace 3B on AWS Trainium2 (automationscribe.com/?p=7116),
"GLA mixer"; these tests check it against results its mathematics fixes
independently of the recurrence (see tests/pins.py).
"""
import json
import os

import numpy as np
import pytest

import pins
from gated_linear_attention_amd import synth
from oracle import c_oracle
from oracle import gla_oracle as orc

TOL = 1e-12


def numpy_impl(q, k, v, lg, S0, cu):
    return orc.recurrent_forward(q, k, v, lg, S0, cu)


def c_impl(q, k, v, lg, S0, cu):
    o, ST, _ = c_oracle.fwd(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                            lg.astype(np.float32), None if S0 is None else S0.astype(np.float32),
                            cu, nthreads=2)
    return o, ST


@pytest.mark.parametrize("name", sorted(pins.ALL_PINS))
def test_numpy_oracle_pin(name):
    e = pins.ALL_PINS[name](numpy_impl)
    assert e <= TOL, f"pin {name}: error {e:.3e}"


@pytest.mark.parametrize("name", sorted(set(pins.ALL_PINS) - {"linearity", "continuation"}))
def test_c_oracle_pin(name):
    # The pins draw fp32-exact inputs, which the C oracle (fp32 inputs, like the
    # library's boundary) reads without rounding. Linearity combines inputs, and
    # continuation feeds back an fp64 state, into values that are not fp32-exact,
    # so those two are checked on the numpy oracle only.
    e = pins.ALL_PINS[name](c_impl)
    assert e <= TOL, f"pin {name}: {e:.3e}"


def test_c_oracle_matches_numpy_tiny_f32():
    w = synth.WORKLOADS["tiny_f32"]
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w)
    o1, S1 = orc.recurrent_forward(q, k, v, lg, S0, cu)
    o2, S2, used = c_oracle.fwd(q, k, v, lg, S0, cu, nthreads=4)
    assert used >= 1
    assert orc.normwise_error(o2, o1) <= TOL
    assert orc.normwise_error(S2, S1) <= TOL


def test_c_oracle_matches_numpy_varlen_bf16():
    w = synth.WORKLOADS["varlen_64"]
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w, H=2, lengths=[70, 1, 0, 130, 64])
    o1, S1 = orc.recurrent_forward(q, k, v, lg, S0, cu)
    o2, S2, _ = c_oracle.fwd(q, k, v, lg, S0, cu, nthreads=3)
    assert orc.normwise_error(o2, o1) <= TOL
    assert orc.normwise_error(S2, S1) <= TOL
    # zero-length sequence: final state is its initial state
    np.testing.assert_array_equal(S2[2], S0[2].astype(np.float64))


def test_c_oracle_thread_count_invariant():
    w = synth.WORKLOADS["train_2k"]
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w, B=2, T=96, H=3)
    o1, S1, _ = c_oracle.fwd(q, k, v, lg, S0, cu, nthreads=1)
    o2, S2, _ = c_oracle.fwd(q, k, v, lg, S0, cu, nthreads=4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_forward_t1_equals_decode_step():
    q, k, v, lg, S0 = pins.rand_inputs(11, B=3, T=1, H=2, dk=4, dv=5)
    o, ST = orc.recurrent_forward(q, k, v, lg, S0)
    od, Sd = orc.decode_step(q[:, 0], k[:, 0], v[:, 0], lg[:, 0], S0)
    assert pins.err(o[:, 0], od) <= TOL
    assert pins.err(ST, Sd) <= TOL


def test_decode_chain_equals_forward():
    steps = 30
    q, k, v, lg, S0 = pins.rand_inputs(12, B=3, T=steps, H=2, dk=4, dv=3)
    o, ST = orc.recurrent_forward(q, k, v, lg, S0)
    S = S0.copy()
    for t in range(steps):
        od, S = orc.decode_step(q[:, t], k[:, t], v[:, t], lg[:, t], S)
        assert pins.err(od, o[:, t]) <= TOL
    assert pins.err(S, ST) <= TOL


def test_c_decode_chain_equals_numpy():
    N, H, dk, dv = 5, 3, 8, 4
    S = synth.make_decode_state(N, H, dk, dv, seed=3).astype(np.float64)
    Sn = S.copy()
    for s in range(10):
        q, k, v, lg = synth.make_decode_step_inputs(N, H, dk, dv, seed=4000 + s)
        oc, _ = c_oracle.decode(q, k, v, lg, S, nthreads=2)
        on, Sn = orc.decode_step(q, k, v, lg, Sn)
        assert orc.normwise_error(oc, on) <= TOL
    assert orc.normwise_error(S, Sn) <= TOL


def test_decode_reset_and_identity_gate():
    N, H, dk, dv = 2, 2, 3, 4
    rng = np.random.default_rng(0)
    q, k, v = rng.standard_normal((N, H, dk)), rng.standard_normal((N, H, dk)), rng.standard_normal((N, H, dv))
    S = rng.standard_normal((N, H, dk, dv))
    o, S1 = orc.decode_step(q, k, v, np.full((N, H), -np.inf), S)
    np.testing.assert_allclose(S1, np.einsum("nhd,nhe->nhde", k, v), rtol=0, atol=0)
    o, S1 = orc.decode_step(q, k, v, np.zeros((N, H)), S)
    np.testing.assert_allclose(S1, S + np.einsum("nhd,nhe->nhde", k, v), rtol=1e-15)
    np.testing.assert_allclose(o, np.einsum("nhd,nhde->nhe", q, S1), rtol=1e-13)


def test_laplace_decay_schedule_matches_printed_values():
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "golden", "laplace_decay_schedule.json")) as f:
        gold = json.load(f)
    lg = synth.laplace_decay_schedule(H=gold["H"], t_min=gold["t_min"], t_max=gold["t_max"])
    lam = np.exp(lg)
    assert lam[0] == pytest.approx(gold["head_0"]["lambda"], abs=1e-15)
    digits = gold["head_15"]["printed_digits"]
    assert round(float(lam[15]), digits) == gold["head_15"]["lambda_printed"]
    # half-life of head h: lambda_h ** half_life == 1/2
    assert lam[15] ** gold["head_15"]["half_life"] == pytest.approx(0.5, rel=1e-12)
    assert np.all(np.diff(lam) > 0)


def test_normwise_error_metric():
    ref = np.array([1.0, -4.0, 2.0])
    assert orc.normwise_error(ref + [0.0, 0.004, 0.0], ref) == pytest.approx(1e-3)
    assert orc.normwise_error(np.array([np.nan, 0, 0]), ref) == float("inf")
    assert orc.normwise_error(np.zeros(0), np.zeros(0)) == 0.0
