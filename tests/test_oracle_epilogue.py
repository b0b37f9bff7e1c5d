"""The fp64 epilogue oracle against its pins, and planted mistakes against the pins.

Each mutant is a copy of the epilogue of Laplace 3B on AWS Trainium2
(automationscribe.com/?p=7116), "GLA mixer", with one plausible mistake; the
pins are strong enough only if every mutant fails at least one of them.
"""
import numpy as np
import pytest

import epilogue_pins as ep
from oracle import epilogue_oracle as eo


@pytest.mark.parametrize("name", list(ep.ALL_PINS))
def test_oracle_passes_pin(name):
    assert ep.ALL_PINS[name](eo.mixer_epilogue) <= 1e-12, name


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def _mutant(o, q, k, v, g, a, rms_w, tier, eps, *, m):
    w = np.asarray(rms_w, np.float64)[np.asarray(tier)]
    if m == "weight_of_head_not_tier":
        w = np.asarray(rms_w, np.float64)[np.arange(len(tier)) % len(rms_w)]
    logit = np.sum(q * a * k, axis=-1, keepdims=True)
    if m == "scale_ignored":
        logit = np.sum(q * k, axis=-1, keepdims=True)
    gate = logit if m == "no_sigmoid" else _sig(logit)
    if m == "sigmoid_of_negated_logit":
        gate = _sig(-logit)
    x = o if m == "augment_after_norm" else o + gate * v
    sg = g * _sig(g)
    if m == "gate_before_norm":
        x = x * sg
    if m == "norm_over_tier":  # one RMS over the concatenated heads of each tier
        ms = np.zeros(x.shape[:-1] + (1,))
        for t in np.unique(tier):
            hs = np.where(np.asarray(tier) == t)[0]
            ms[:, hs] = np.mean(x[:, hs] ** 2, axis=(-2, -1), keepdims=True)
    else:
        ms = np.mean(x * x, axis=-1, keepdims=True)
    if m == "norm_without_sqrt":
        y = x / (ms + eps) * w
    elif m == "eps_outside_sqrt":
        y = x / (np.sqrt(ms) + eps) * w
    else:
        y = x / np.sqrt(ms + eps) * w
    if m == "augment_after_norm":
        y = y + gate * v
    if m == "gate_before_norm":
        return y
    if m == "sigmoid_output_gate":
        return y * _sig(g)
    return y * sg


MUTANTS = ["no_sigmoid", "scale_ignored", "sigmoid_of_negated_logit", "augment_after_norm",
           "gate_before_norm", "norm_over_tier", "norm_without_sqrt", "eps_outside_sqrt",
           "weight_of_head_not_tier", "sigmoid_output_gate"]


def test_unmutated_copy_passes():
    for name, pin in ep.ALL_PINS.items():
        assert pin(lambda *a: _mutant(*a, m=None)) <= 1e-12, name


@pytest.mark.parametrize("m", MUTANTS)
def test_mutant_is_caught(m):
    caught = [name for name, pin in ep.ALL_PINS.items()
              if not pin(lambda *a: _mutant(*a, m=m)) <= 1e-6]
    assert caught, f"mutant {m} passed every pin"
