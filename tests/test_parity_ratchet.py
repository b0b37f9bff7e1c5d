"""Error ratchet of the benchmarked configs (CPU; reads committed records).

tests/parity_record.json holds, per benchmarked config and output tensor, the
largest normwise error per (sequence, head) pair against the fp64 oracle that
bench.py measured on MI355X (its JSON line's 'parity' object). Checked here:
  * every recorded error is within its bar (2e-3 for the bf16-input configs);
  * a newer bench record in the repository (BENCH_r*.json files holding that
    line) may not regress: each error must stay at or below
    max(FLOOR, 1.05 x the recorded one). The kernels are deterministic, so an
    unchanged build reproduces its errors exactly; a change that moves them up
    by more than 5% must justify it and lower or raise the record explicitly.
"""
import glob
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORD = os.path.join(ROOT, "tests", "parity_record.json")
FLOOR = 1e-6          # below this, differences are rounding noise of the error itself
BAR = 2e-3            # bf16 inputs, fp32 accumulation (every benchmarked config)
ALLOWED_GROWTH = 1.05


def _record():
    with open(RECORD) as f:
        return json.load(f)["errors"]


def test_record_within_bars():
    rec = _record()
    assert rec, "empty parity record"
    for cfg, errs in rec.items():
        assert errs, cfg
        for name, e in errs.items():
            assert 0.0 <= e <= BAR, (cfg, name, e)


def _bench_lines():
    """(path, parsed JSON line) of the bench records in the repository that
    carry a 'parity' object, oldest first."""
    out = []
    for path in sorted(glob.glob(os.path.join(ROOT, "BENCH_r*.json"))):
        try:
            with open(path) as f:
                rec = json.load(f)
        except (OSError, ValueError):
            continue
        line = rec.get("parsed") if isinstance(rec, dict) else None
        if isinstance(line, dict) and isinstance(line.get("parity"), dict):
            out.append((path, line))
    return out


def ratchet_violations(record, parity):
    """Entries of a bench line's parity object above max(FLOOR, 1.05 x record)."""
    bad = []
    for cfg, errs in parity.items():
        for name, e in errs.items():
            if not isinstance(e, float) or name not in record.get(cfg, {}):
                continue
            limit = max(FLOOR, ALLOWED_GROWTH * record[cfg][name])
            if e > limit:
                bad.append((cfg, name, e, limit))
    return bad


def test_newest_bench_record_does_not_regress():
    lines = _bench_lines()
    if not lines:
        pytest.skip("no bench record with a parity object in the repository yet")
    path, line = lines[-1]
    assert ratchet_violations(_record(), line["parity"]) == [], path


def test_ratchet_catches_a_regression():
    rec = _record()
    cfg = next(iter(rec))
    name = next(iter(rec[cfg]))
    worse = {cfg: {name: max(FLOOR, rec[cfg][name]) * 1.2}}
    same = {cfg: {name: rec[cfg][name]}}
    assert ratchet_violations(rec, worse) and not ratchet_violations(rec, same)
