"""Pins of the oracle's backward (oracle.gla_oracle.recurrent_backward).

The backward is the reverse-mode adjoint of the recurrence, written out by
hand. It is pinned here to two things that do not share that derivation:
  * central finite differences of the forward oracle (the gradient's
    definition), on tiny dense and packed inputs;
  * fp64 automatic differentiation (torch.autograd) of an independent forward
    written in this file with torch ops;
plus the gate identity the GPU backward relies on, and planted mistakes in a
copy of the backward that the finite-difference pin must catch.
"""
import numpy as np
import pytest
import torch

from oracle import gla_oracle as G


def _inputs(seed, B, T, H, dk, dv, cu=None, s0=True, dst=True, reset_at=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk)) / np.sqrt(dk)
    v = rng.standard_normal((B, T, H, dv))
    lg = np.log(rng.uniform(0.3, 0.99, (B, T, H)))
    if reset_at is not None:
        lg[:, reset_at, :] = -np.inf
    N = B if cu is None else len(cu) - 1
    S0 = rng.standard_normal((N, H, dk, dv)) if s0 else None
    dO = rng.standard_normal((B, T, H, dv))
    dS_T = rng.standard_normal((N, H, dk, dv)) if dst else None
    return q, k, v, lg, S0, dO, dS_T


def _loss(q, k, v, lg, S0, dO, dS_T, cu):
    o, ST = G.recurrent_forward(q, k, v, lg, S0, cu)
    val = np.sum(o * dO)
    if dS_T is not None:
        val += np.sum(ST * dS_T)
    return val


def _finite_differences(q, k, v, lg, S0, dO, dS_T, cu, eps=1e-6):
    out = []
    args = dict(q=q, k=k, v=v, lg=lg, S0=S0)
    for name in ("q", "k", "v", "lg", "S0"):
        a = args[name]
        if a is None:
            out.append(None)
            continue
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            if not np.isfinite(a[idx]):
                continue
            hi, lo = a.copy(), a.copy()
            hi[idx] += eps
            lo[idx] -= eps
            a_hi = dict(args, **{name: hi})
            a_lo = dict(args, **{name: lo})
            fd[idx] = (_loss(**a_hi, dO=dO, dS_T=dS_T, cu=cu) -
                       _loss(**a_lo, dO=dO, dS_T=dS_T, cu=cu)) / (2 * eps)
        out.append(fd)
    return out


CASES = [
    dict(seed=1, B=1, T=6, H=1, dk=3, dv=2),
    dict(seed=2, B=2, T=5, H=2, dk=2, dv=3, s0=False),
    dict(seed=3, B=1, T=7, H=1, dk=2, dv=2, cu=[0, 3, 3, 7], dst=False),
    dict(seed=4, B=1, T=6, H=1, dk=2, dv=2, reset_at=3),
]


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_finite_differences(case):
    cu = case.get("cu")
    q, k, v, lg, S0, dO, dS_T = _inputs(**{kk: vv for kk, vv in case.items()})
    got = G.recurrent_backward(q, k, v, lg, dO, dS_T, S0, cu)
    fds = _finite_differences(q, k, v, lg, S0, dO, dS_T, cu)
    for name, g, fd in zip(("dq", "dk", "dv", "dlog_g", "dS0"), got, fds):
        if fd is None:
            continue
        mask = np.isfinite(lg) if name == "dlog_g" else np.ones(fd.shape, bool)
        err = np.abs(g - fd)[mask].max() / max(np.abs(fd[mask]).max(), 1e-300)
        assert err < 1e-7, (name, err)


def _torch_forward(q, k, v, lg, S0, cu):
    """An independent forward in torch ops (differentiable), same definition."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bounds = [(b, 0, T) for b in range(B)] if cu is None else \
        [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    outs = [[None] * T for _ in range(B)]
    finals = []
    for n, (b, s, e) in enumerate(bounds):
        S = torch.zeros(H, dk, dv, dtype=torch.float64) if S0 is None else S0[n]
        for t in range(s, e):
            S = torch.exp(lg[b, t])[:, None, None] * S + k[b, t][:, :, None] * v[b, t][:, None, :]
            outs[b][t] = (q[b, t][:, :, None] * S).sum(1)
        finals.append(S)
    zero = torch.zeros(H, dv, dtype=torch.float64)
    o = torch.stack([torch.stack([x if x is not None else zero for x in row]) for row in outs])
    return o, torch.stack(finals)


@pytest.mark.parametrize("cu", [None, [0, 5, 6, 6, 19]])
def test_backward_matches_autograd(cu):
    B = 2 if cu is None else 1
    T = 19
    q, k, v, lg, S0, dO, dS_T = _inputs(11, B, T, 2, 4, 3, cu=cu)
    tq, tk, tv, tlg, tS0 = (torch.tensor(a, dtype=torch.float64, requires_grad=True)
                            for a in (q, k, v, lg, S0))
    o, ST = _torch_forward(tq, tk, tv, tlg, tS0, cu)
    loss = (o * torch.tensor(dO)).sum() + (ST * torch.tensor(dS_T)).sum()
    loss.backward()
    got = G.recurrent_backward(q, k, v, lg, dO, dS_T, S0, cu)
    for g, ref in zip(got, (tq.grad, tk.grad, tv.grad, tlg.grad, tS0.grad)):
        ref = ref.numpy()
        assert np.abs(g - ref).max() <= 1e-11 * max(np.abs(ref).max(), 1.0)


def test_gate_gradient_identity():
    """d L / d B_u = q_u . dq_u - k_u . dk_u (+ <dS_T, S_T> at a sequence's last
    token), B the cumulative log-gate, so dlog_g is its reverse cumulative sum
    within each sequence: the identity the GPU backward computes dlog_g from."""
    cu = [0, 4, 9, 9, 12]
    q, k, v, lg, S0, dO, dS_T = _inputs(21, 1, 12, 2, 3, 4, cu=cu)
    dq, dk, dv, dl, dS0 = G.recurrent_backward(q, k, v, lg, dO, dS_T, S0, cu)
    _, ST = G.recurrent_forward(q, k, v, lg, S0, cu)
    dB = np.einsum("bthd,bthd->bth", q, dq) - np.einsum("bthd,bthd->bth", k, dk)
    for n in range(len(cu) - 1):
        s, e = cu[n], cu[n + 1]
        if e > s:
            dB[0, e - 1] += np.einsum("hde,hde->h", dS_T[n], ST[n])
            ref = np.cumsum(dB[0, s:e][::-1], axis=0)[::-1]
            np.testing.assert_allclose(dl[0, s:e], ref, rtol=1e-11, atol=1e-11)


def test_reset_gate_blocks_gradient_flow():
    """l_t = -inf zeroes the state: nothing before t reaches outputs at or after
    t, so dO at or after t changes no gradient of an earlier token, and the
    reset token's own dlog_g is 0 (g = 0)."""
    q, k, v, lg, S0, dO, dS_T = _inputs(31, 1, 8, 1, 3, 2, reset_at=4)
    base = G.recurrent_backward(q, k, v, lg, dO, dS_T, S0)
    dO2 = dO.copy()
    dO2[:, 4:] = np.random.default_rng(5).standard_normal(dO2[:, 4:].shape)
    dS_T2 = dS_T + 1.0
    other = G.recurrent_backward(q, k, v, lg, dO2, dS_T2, S0)
    for a, b in zip(base[:3], other[:3]):
        np.testing.assert_array_equal(a[:, :4], b[:, :4])
    assert base[3][0, 4, 0] == 0.0
    np.testing.assert_array_equal(base[4], other[4])


def _mutant_backward(q, k, v, lg, dO, dS_T, S0, mutation):
    """A copy of the oracle's backward walk with one planted mistake."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = [np.zeros((B, T, H, dk)), np.zeros((B, T, H, dk)), np.zeros((B, T, H, dv)),
           np.zeros((B, T, H)), np.zeros((B, H, dk, dv))]
    for b in range(B):
        for h in range(H):
            S = S0[b, h].copy()
            states = [S]
            for t in range(T):
                S = np.exp(lg[b, t, h]) * S + np.outer(k[b, t, h], v[b, t, h])
                states.append(S)
            A = dS_T[b, h].copy()
            for t in range(T - 1, -1, -1):
                g = np.exp(lg[b, t, h])
                if mutation != "readout_adjoint_after_use":
                    A = A + np.outer(q[b, t, h], dO[b, t, h])
                out[0][b, t, h] = (states[t] if mutation == "dq_from_old_state" else states[t + 1]) @ dO[b, t, h]
                out[1][b, t, h] = A @ v[b, t, h]
                # dv_t = k_t A; the mutant uses the adjoint transposed (dk == dv here)
                out[2][b, t, h] = (A @ k[b, t, h]) if mutation == "dv_transposed_adjoint" else (A.T @ k[b, t, h])
                dl = np.sum(A * states[t])
                out[3][b, t, h] = dl if mutation == "dlog_g_without_gate" else g * dl
                if mutation == "readout_adjoint_after_use":
                    A = A + np.outer(q[b, t, h], dO[b, t, h])
                A = A if mutation == "adjoint_not_decayed" else g * A
            out[4][b, h] = A
    return out


@pytest.mark.parametrize("mutation", ["dq_from_old_state", "dlog_g_without_gate",
                                      "readout_adjoint_after_use", "adjoint_not_decayed",
                                      "dv_transposed_adjoint"])
def test_backward_mutants_fail_the_pin(mutation):
    q, k, v, lg, S0, dO, dS_T = _inputs(41, 1, 5, 1, 3, 3)
    ref = _mutant_backward(q, k, v, lg, dO, dS_T, S0, None)
    good = G.recurrent_backward(q, k, v, lg, dO, dS_T, S0)
    for a, b in zip(ref, good):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    bad = _mutant_backward(q, k, v, lg, dO, dS_T, S0, mutation)
    fds = _finite_differences(q, k, v, lg, S0, dO, dS_T, None)
    worst = max(np.abs(g - fd).max() / np.abs(fd).max() for g, fd in zip(bad, fds))
    assert worst > 1e-3, mutation


@pytest.mark.parametrize("cu,reset_at,s0,dst", [
    (None, None, True, True),
    (None, 4, False, True),
    (np.array([0, 0, 9, 10, 23], dtype=np.int64), 11, True, False),
])
def test_c_backward_matches_numpy(cu, reset_at, s0, dst):
    """The C oracle's backward (oracle/gla_oracle.c, used at full sizes) is a
    second, independent transcription of the adjoint walk: it must give the
    numpy backward's gradients, which the finite-difference and autograd pins
    above hold to the definition, to fp64 rounding (dense and packed batches,
    an empty sequence, a reset gate, with and without S0 and dS_T)."""
    from oracle import c_oracle
    B = 2 if cu is None else 1
    T = 23
    q, k, v, lg, S0, dO, dS_T = _inputs(31, B, T, 3, 8, 6, cu=cu, s0=s0, dst=dst,
                                        reset_at=reset_at)
    f32 = lambda a: None if a is None else a.astype(np.float32)
    q, k, v, lg, S0, dO, dS_T = (f32(x) for x in (q, k, v, lg, S0, dO, dS_T))
    ref = G.recurrent_backward(q, k, v, lg, dO, dS_T, S0, cu)
    got = c_oracle.bwd(q, k, v, lg, dO, dS_T, S0, cu, nthreads=3)[:5]
    for g, r in zip(got, ref):
        assert g.shape == r.shape
        assert np.abs(g - r).max() <= 1e-12 * max(1.0, np.abs(r).max())
