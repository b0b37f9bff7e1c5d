"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant below is the token-by-token recurrence of the oracle with one
plausible mistake (dropped term, wrong sign, wrong index, transposed
operand, wrong order of update and readout). The pins of tests/pins.py are
strong enough only if every mutant fails one of them.
"""
import numpy as np
import pytest

import pins


def _recurrence(q, k, v, lg, S0, cu, *, mutation=None):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu is None:
        bounds = [(b, 0, T) for b in range(B)]
    else:
        bounds = [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((len(bounds), H, dk, dv))
    S = None
    for n, (b, s0, s1) in enumerate(bounds):
        if mutation == "no_reset_between_sequences" and S is not None:
            pass
        elif S0 is None or mutation == "drop_S0":
            S = np.zeros((H, dk, dv))
        else:
            S = np.array(S0[n], dtype=np.float64)
        for t in range(s0, s1):
            tg = t
            if mutation == "gate_of_next_token":
                tg = min(t + 1, s1 - 1)
            g = np.exp(lg[b, tg])[:, None, None]
            if mutation == "gate_not_exponentiated":
                g = lg[b, tg][:, None, None]
            kv = np.einsum("hd,he->hde", k[b, t], v[b, t])
            if mutation == "readout_before_update":
                o[b, t] = np.einsum("hd,hde->he", q[b, t], S)
            if mutation == "gate_after_add":
                S = g * (S + kv)
            elif mutation == "minus_kv":
                S = g * S - kv
            elif mutation == "value_key_swapped":
                S = g * S + np.einsum("hd,he->hde", v[b, t][:, :dk], k[b, t][:, :dv]) if dk == dv else g * S + kv * 1.01
            else:
                S = g * S + kv
            if mutation == "readout_before_update":
                continue
            if mutation == "transposed_readout":
                o[b, t] = np.einsum("hd,hed->he", q[b, t], S) if dk == dv else 0.99 * np.einsum("hd,hde->he", q[b, t], S)
            elif mutation == "readout_uses_key":
                o[b, t] = np.einsum("hd,hde->he", k[b, t], S)
            else:
                o[b, t] = np.einsum("hd,hde->he", q[b, t], S)
        ST[n] = S
    return o, ST


MUTATIONS = [
    "readout_before_update",
    "gate_after_add",
    "drop_S0",
    "minus_kv",
    "gate_of_next_token",
    "gate_not_exponentiated",
    "transposed_readout",
    "readout_uses_key",
    "value_key_swapped",
    "no_reset_between_sequences",
]


def test_unmutated_copy_passes_all_pins():
    impl = lambda *a: _recurrence(*a)
    for name, pin in pins.ALL_PINS.items():
        assert pin(impl) <= 1e-12, name


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_mutant_is_caught(mutation):
    impl = lambda *a: _recurrence(*a, mutation=mutation)
    failures = []
    for name, pin in pins.ALL_PINS.items():
        try:
            e = pin(impl)
        except Exception as exc:  # a crash also counts as caught
            failures.append((name, repr(exc)))
            continue
        if not (e <= 1e-6):
            failures.append((name, e))
    assert failures, f"mutant {mutation} passed every pin"
