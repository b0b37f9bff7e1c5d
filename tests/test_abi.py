"""The C ABI library loads and exports every symbol include/gla.h declares;
host-side argument checks return their status codes without touching the GPU."""
import ctypes
import os
import re

import pytest

from gated_linear_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "gla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gla_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    assert header_functions() == ["gla_bwd_chunked", "gla_bwd_chunked_workspace_size",
                                  "gla_decode_mixer", "gla_decode_slot_order", "gla_decode_step",
                                  "gla_decode_step_slots",
                                  "gla_fwd_chunked",
                                  "gla_fwd_chunked_fixed_decay",
                                  "gla_fwd_chunked_noalloc",
                                  "gla_fwd_chunked_noalloc_max_scratch",
                                  "gla_fwd_chunked_workspace_size", "gla_mixer_epilogue",
                                  "gla_status_string"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code, name in [(0, "GLA_OK"), (1, "GLA_ERR_INVALID_ARGUMENT"), (2, "GLA_ERR_UNSUPPORTED"),
                       (3, "GLA_ERR_WORKSPACE"), (4, "GLA_ERR_HIP")]:
        assert _lib.status_string(code) == name
    assert _lib.status_string(99) == "GLA_UNKNOWN_STATUS"


def _fwd(fixed=False, **kw):
    a = dict(q=None, k=None, v=None, g=None, S0=None, cu=None, o=None, ST=None, B=1, T=64, H=1,
             dk=64, dv=64, N=1, C=64, ind=_lib.GLA_BF16, outd=_lib.GLA_F32, ws=None, wsb=0)
    a.update(kw)
    lib = _lib.load()
    fn = lib.gla_fwd_chunked_fixed_decay if fixed else lib.gla_fwd_chunked
    return fn(a["q"], a["k"], a["v"], a["g"], a["S0"], a["cu"], a["o"], a["ST"], a["B"], a["T"],
              a["H"], a["dk"], a["dv"], a["N"], a["C"], a["ind"], a["outd"], a["ws"], a["wsb"],
              None)


FAKE = 1 << 40  # never dereferenced: every call below fails validation first


def test_fwd_rejects_bad_arguments_before_launch():
    P = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30),
             o=FAKE + (4 << 30))
    assert _fwd(B=-1, **P) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert _fwd(ind=7, **P) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert _fwd(N=2, **P) == _lib.GLA_ERR_INVALID_ARGUMENT            # N != B without cu
    assert _fwd(dk=96, **P) == _lib.GLA_ERR_UNSUPPORTED
    assert _fwd(dv=192, **P) == _lib.GLA_ERR_UNSUPPORTED
    assert _fwd(dk=192, dv=96, **P) == _lib.GLA_ERR_UNSUPPORTED
    assert _fwd(dk=96, dv=192, B=0, N=0, **P) == _lib.GLA_OK  # the Laplace head shape is accepted
    assert _fwd(C=32, **P) == _lib.GLA_ERR_UNSUPPORTED
    assert _fwd(C=512, **P) == _lib.GLA_ERR_UNSUPPORTED
    assert _fwd(C=256, H=0, **P) == _lib.GLA_OK  # 256-token chunks are accepted
    assert _fwd(**{**P, "q": None}) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert _fwd(**{**P, "o": P["q"] + 64}) == _lib.GLA_ERR_INVALID_ARGUMENT  # o overlaps q
    assert _fwd(cu=FAKE + (5 << 30), B=2, N=2, **P) == _lib.GLA_ERR_INVALID_ARGUMENT
    # zero heads or zero sequences: nothing to do
    assert _fwd(H=0, **P) == _lib.GLA_OK
    assert _fwd(B=0, N=0, **P) == _lib.GLA_OK


def test_fixed_decay_fwd_rejects_bad_arguments_before_launch():
    P = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30),
             o=FAKE + (4 << 30), H=8)
    assert _fwd(True, B=-1, **P) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert _fwd(True, dk=96, **P) == _lib.GLA_ERR_UNSUPPORTED
    assert _fwd(True, C=512, **P) == _lib.GLA_ERR_UNSUPPORTED
    assert _fwd(True, **{**P, "g": None}) == _lib.GLA_ERR_INVALID_ARGUMENT
    # log_lambda holds H = 8 floats: an o that starts at its fifth overlaps it
    assert _fwd(True, **{**P, "o": P["g"] + 16}) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert _fwd(True, H=0, **{k: v for k, v in P.items() if k != "H"}) == _lib.GLA_OK


def test_fwd_requires_workspace_when_planned():
    lib = _lib.load()
    n = lib.gla_fwd_chunked_workspace_size(1, 4096, 1, 64, 64, 3, 64, 1, _lib.GLA_BF16)
    assert n > 0
    P = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30),
             o=FAKE + (4 << 30), cu=FAKE + (5 << 30))
    assert _fwd(B=1, T=4096, N=3, ws=None, wsb=0, **P) == _lib.GLA_ERR_WORKSPACE
    assert _fwd(B=1, T=4096, N=3, ws=FAKE + (6 << 30), wsb=n - 1, **P) == _lib.GLA_ERR_WORKSPACE


def test_workspace_size_is_zero_for_whole_sequences():
    lib = _lib.load()
    # 8 x 16 heads x 2 slices = 256 work units covers the device: no split, no plan
    assert lib.gla_fwd_chunked_workspace_size(8, 2048, 16, 128, 128, 8, 64, 0, _lib.GLA_BF16) == 0
    assert lib.gla_fwd_chunked_workspace_size(1, 256, 2, 64, 64, 1, 64, 0, 7) == 0


def test_decode_rejects_bad_arguments_before_launch():
    lib = _lib.load()
    base = [FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30),
            FAKE + (5 << 30)]
    call = lambda ptrs, N=4, H=2, dk=64, dv=64, ind=_lib.GLA_BF16: lib.gla_decode_step(
        *ptrs, N, H, dk, dv, ind, _lib.GLA_F32, None)
    assert call(base, N=-1) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(base, dk=96) == _lib.GLA_ERR_UNSUPPORTED
    assert call(base, dk=192, dv=96) == _lib.GLA_ERR_UNSUPPORTED
    assert call(base, dk=96, dv=192, N=0) == _lib.GLA_OK  # the Laplace head shape is accepted
    assert call(base, ind=5) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call([None] + base[1:]) == _lib.GLA_ERR_INVALID_ARGUMENT
    bad = list(base)
    bad[5] = base[4] + 16  # o inside S
    assert call(bad) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(base, N=0) == _lib.GLA_OK


def _bwd(**kw):
    a = dict(q=None, k=None, v=None, g=None, S0=None, cu=None, dO=None, dST=None, dq=None,
             dk=None, dv=None, dg=None, dS0=None, B=1, T=64, H=1, dkd=64, dvd=64, N=1, C=64,
             ind=_lib.GLA_BF16, ws=None, wsb=0)
    a.update(kw)
    return _lib.load().gla_bwd_chunked(a["q"], a["k"], a["v"], a["g"], a["S0"], a["cu"], a["dO"],
                                       a["dST"], a["dq"], a["dk"], a["dv"], a["dg"], a["dS0"],
                                       a["B"], a["T"], a["H"], a["dkd"], a["dvd"], a["N"], a["C"],
                                       a["ind"], a["ws"], a["wsb"], None)


def test_bwd_rejects_bad_arguments_before_launch():
    G = 1 << 30
    P = dict(q=FAKE, k=FAKE + G, v=FAKE + 2 * G, g=FAKE + 3 * G, dO=FAKE + 4 * G,
             dq=FAKE + 5 * G, dk=FAKE + 6 * G, dv=FAKE + 7 * G, dg=FAKE + 8 * G)
    lib = _lib.load()
    n = lib.gla_bwd_chunked_workspace_size(1, 64, 1, 64, 64, 1, 64, 0, _lib.GLA_BF16)
    assert n > 0  # transposed states and per-token partial sums live in the workspace
    W = dict(ws=FAKE + 9 * G, wsb=n)
    assert _bwd(B=-1, **P, **W) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert _bwd(ind=5, **P, **W) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert _bwd(N=2, **P, **W) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert _bwd(dkd=96, **P, **W) == _lib.GLA_ERR_UNSUPPORTED
    assert _bwd(C=512, **P, **W) == _lib.GLA_ERR_UNSUPPORTED
    assert _bwd(**{**P, "dO": None}, **W) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert _bwd(**{**P, "dg": None}, **W) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert _bwd(**{**P, "dq": P["q"] + 64}, **W) == _lib.GLA_ERR_INVALID_ARGUMENT  # output on input
    assert _bwd(**{**P, "dk": P["dq"] + 64}, **W) == _lib.GLA_ERR_INVALID_ARGUMENT  # outputs overlap
    assert _bwd(**P) == _lib.GLA_ERR_WORKSPACE
    assert _bwd(**P, ws=FAKE + 9 * G, wsb=n - 1) == _lib.GLA_ERR_WORKSPACE
    assert _bwd(H=0, **P) == _lib.GLA_OK
    assert lib.gla_bwd_chunked_workspace_size(1, 64, 1, 96, 64, 1, 64, 0, _lib.GLA_BF16) == 0
    # Laplace 3B's 96 x 192 heads are supported; their transpose 192 x 96 is not
    assert lib.gla_bwd_chunked_workspace_size(1, 64, 1, 96, 192, 1, 64, 0, _lib.GLA_BF16) > 0
    assert lib.gla_bwd_chunked_workspace_size(1, 64, 1, 192, 96, 1, 64, 0, _lib.GLA_BF16) == 0
    assert _bwd(dkd=192, dvd=96, **P, **W) == _lib.GLA_ERR_UNSUPPORTED


def test_decode_slots_rejects_bad_arguments_before_launch():
    G = 1 << 30
    lib = _lib.load()
    def call(q=FAKE, k=FAKE + G, v=FAKE + 2 * G, g=FAKE + 3 * G, S=FAKE + 4 * G,
             slots=FAKE + 40 * G, o=FAKE + 41 * G, N=4, P=8, H=2, dk=64, dv=64,
             ind=_lib.GLA_BF16, outd=_lib.GLA_F32, order=None):
        return lib.gla_decode_step_slots(q, k, v, g, S, slots, order, o, N, P, H, dk, dv, ind,
                                         outd, None)
    assert call(N=-1) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(P=-1) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(ind=3) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(dk=96) == _lib.GLA_ERR_UNSUPPORTED
    assert call(slots=None) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(S=None) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(o=FAKE + 4 * G + 64) == _lib.GLA_ERR_INVALID_ARGUMENT   # o inside the pool
    assert call(slots=FAKE + 4 * G + 64) == _lib.GLA_ERR_INVALID_ARGUMENT  # slots inside the pool
    assert call(order=FAKE + 4 * G + 64) == _lib.GLA_ERR_INVALID_ARGUMENT  # order inside the pool
    assert call(order=FAKE + 41 * G) == _lib.GLA_ERR_INVALID_ARGUMENT      # order under o
    assert call(order=FAKE + 42 * G + 2) == _lib.GLA_ERR_INVALID_ARGUMENT  # misaligned
    assert call(N=0) == _lib.GLA_OK
    assert call(N=0, order=FAKE + 42 * G) == _lib.GLA_OK


def test_slot_order_rejects_bad_arguments_before_launch():
    lib = _lib.load()
    G = 1 << 30
    S, O = FAKE, FAKE + G
    call = lambda s=S, n=4, P=8, o=O, b=1 << 20: lib.gla_decode_slot_order(s, n, P, b, o, None)
    assert call(n=-1) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(P=-1) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(P=32769) == _lib.GLA_ERR_UNSUPPORTED   # one LDS counter per pool entry
    assert call(s=None) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(o=None) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(o=S + 8) == _lib.GLA_ERR_INVALID_ARGUMENT   # order over the slots
    assert call(o=O + 2) == _lib.GLA_ERR_INVALID_ARGUMENT   # misaligned
    assert call(n=0, s=None, o=None) == _lib.GLA_OK


def test_epilogue_rejects_bad_arguments_before_launch():
    lib = _lib.load()
    P = [FAKE + (i << 30) for i in range(7)]  # o, q, k, v, g, a, rms_w
    Z = FAKE + (8 << 30)
    F32, BF = _lib.GLA_F32, _lib.GLA_BF16
    call = lambda p=P, z=Z, eps=1e-6, n=16, H=2, dk=64, dv=64, od=F32, ind=BF, outd=F32: \
        lib.gla_mixer_epilogue(*p, eps, z, n, H, dk, dv, od, ind, outd, None)
    assert call(n=-1) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(od=3) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(eps=-1.0) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(eps=float("nan")) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(eps=float("inf")) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(dk=96) == _lib.GLA_ERR_UNSUPPORTED
    assert call(dk=96, dv=192, n=0) == _lib.GLA_OK
    assert call(p=[None] + P[1:]) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(z=None) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(z=P[1] + 64) == _lib.GLA_ERR_INVALID_ARGUMENT      # z overlaps q
    assert call(z=P[5]) == _lib.GLA_ERR_INVALID_ARGUMENT           # z overlaps a
    assert call(z=P[0] + 16) == _lib.GLA_ERR_INVALID_ARGUMENT      # z partly over o
    assert call(z=P[0], outd=BF) == _lib.GLA_ERR_INVALID_ARGUMENT  # in place needs o's dtype
    assert call(H=0) == _lib.GLA_OK


def test_decode_mixer_rejects_bad_arguments_before_launch():
    lib = _lib.load()
    F32, BF = _lib.GLA_F32, _lib.GLA_BF16
    q, k, v, g, S, go, a, w, z = (FAKE + (i << 30) for i in range(9))

    def call(N=4, H=2, dk=64, dv=64, eps=1e-6, slots=None, P=0, zz=None, ind=BF, ptrs=None,
             order=None):
        p = ptrs or (q, k, v, g, S)
        return lib.gla_decode_mixer(*p, slots, order, P, go, a, w, eps, zz or z, N, H, dk, dv,
                                    ind, F32, None)
    assert call(N=-1) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(eps=-1.0) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(ind=9) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(dk=96) == _lib.GLA_ERR_UNSUPPORTED
    assert call(dk=96, dv=192, N=0) == _lib.GLA_OK
    assert call(slots=FAKE + (10 << 30), P=-1) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(ptrs=(None, k, v, g, S)) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(zz=S + 64) == _lib.GLA_ERR_INVALID_ARGUMENT       # z inside the state
    assert call(zz=go) == _lib.GLA_ERR_INVALID_ARGUMENT           # z over the gate stream
    assert call(ptrs=(q, k, v, g, q + 16)) == _lib.GLA_ERR_INVALID_ARGUMENT  # S over q
    assert call(order=FAKE + (11 << 30)) == _lib.GLA_ERR_INVALID_ARGUMENT   # order without slots
    assert call(slots=FAKE + (10 << 30), P=8, order=S + 64) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(H=0) == _lib.GLA_OK



def test_misaligned_pointers_rejected_before_launch():
    """Tensors need 16-byte alignment (4 bytes for the log-gate streams and the
    int32 arrays); each entry point refuses an offset pointer, and accepts the
    scalar streams at 4-byte offsets."""
    lib = _lib.load()
    G = 1 << 30
    BAD = _lib.GLA_ERR_INVALID_ARGUMENT
    F32, BF = _lib.GLA_F32, _lib.GLA_BF16
    P = dict(q=FAKE, k=FAKE + G, v=FAKE + 2 * G, g=FAKE + 3 * G, o=FAKE + 4 * G, H=0)
    # H = 0 returns before launching anything, but after the pointer checks
    assert _fwd(**P) == _lib.GLA_OK
    for name, off in [("q", 2), ("k", 8), ("v", 4), ("o", 8), ("S0", 4), ("ST", 12)]:
        base = P.get(name, FAKE + 5 * G)
        kw = {**P, name: base + off}
        assert _fwd(**kw) == BAD, name
        assert _fwd(True, **kw) == BAD, name
    assert _fwd(**{**P, "g": P["g"] + 4}) == _lib.GLA_OK      # gates: 4-byte alignment
    assert _fwd(**{**P, "g": P["g"] + 2}) == BAD
    assert _fwd(**{**P, "cu": FAKE + 6 * G + 4, "B": 1, "N": 1}) == _lib.GLA_OK
    assert _fwd(**{**P, "cu": FAKE + 6 * G + 2, "B": 1, "N": 1}) == BAD
    assert _fwd(**{**P, "ws": FAKE + 7 * G + 8, "wsb": 1 << 20}) == BAD

    B = dict(q=FAKE, k=FAKE + G, v=FAKE + 2 * G, g=FAKE + 3 * G, dO=FAKE + 4 * G,
             dq=FAKE + 5 * G, dk=FAKE + 6 * G, dv=FAKE + 7 * G, dg=FAKE + 8 * G, H=0)
    assert _bwd(**B) == _lib.GLA_OK
    for name in ["q", "k", "v", "dO", "dq", "dk", "dv"]:
        assert _bwd(**{**B, name: B[name] + 8}) == BAD, name
    assert _bwd(**{**B, "dS0": FAKE + 9 * G + 4}) == BAD
    assert _bwd(**{**B, "dg": B["dg"] + 4}) == _lib.GLA_OK
    assert _bwd(**{**B, "dg": B["dg"] + 1}) == BAD

    ptr = [FAKE + i * G for i in range(6)]  # q, k, v, g, S, o
    dec = lambda p: lib.gla_decode_step(*p, 4, 2, 64, 64, BF, F32, None)
    for i in [0, 1, 2, 4, 5]:
        assert dec([x + 8 * (j == i) for j, x in enumerate(ptr)]) == BAD, i
    slots = FAKE + 40 * G
    dsl = lambda p, s: lib.gla_decode_step_slots(*p[:5], s, None, p[5], 4, 8, 2, 64, 64, BF, F32,
                                                 None)
    assert dsl(ptr, slots + 2) == BAD
    assert dsl([x + 8 * (j == 4) for j, x in enumerate(ptr)], slots) == BAD  # the pool

    E = [FAKE + (i << 30) for i in range(7)]  # o, q, k, v, g, a, rms_w
    epi = lambda p, z: lib.gla_mixer_epilogue(*p, 1e-6, z, 16, 2, 64, 64, F32, BF, F32, None)
    for i in range(7):
        assert epi([x + 8 * (j == i) for j, x in enumerate(E)], FAKE + (8 << 30)) == BAD, i
    assert epi(E, FAKE + (8 << 30) + 4) == BAD

    q, k, v, g, S, go, a, w, z = (FAKE + (i << 30) for i in range(9))
    mix = lambda q=q, S=S, go=go, z=z, g=g: lib.gla_decode_mixer(
        q, k, v, g, S, None, None, 0, go, a, w, 1e-6, z, 4, 2, 64, 64, BF, F32, None)
    assert mix(q=q + 8) == BAD and mix(S=S + 4) == BAD and mix(go=go + 2) == BAD
    assert mix(z=z + 8) == BAD and mix(g=g + 2) == BAD


def test_binding_refuses_host_tensors():
    """The binding hands only device memory to the library: host tensors are
    refused before any call into it."""
    import torch
    import gated_linear_attention_amd as gla
    q = torch.zeros((1, 64, 1, 64), dtype=torch.bfloat16)
    g = torch.zeros((1, 64, 1), dtype=torch.float32)
    for call in (lambda: gla.fwd_chunked(q, q, q, g),
                 lambda: gla.decode_step(q[0], q[0], q[0], g[0], torch.zeros((64, 1, 64, 64))),
                 lambda: gla.bwd_chunked(q, q, q, g, q)):
        with pytest.raises(ValueError, match="GPU memory"):
            call()


def test_noalloc_forward_checks_before_any_launch():
    """gla_fwd_chunked_noalloc: the forward's argument checks, then its fixed
    scratch: a call that needs more than the library holds is refused with
    GLA_ERR_WORKSPACE before anything is enqueued (host logic only: no call
    here reaches the GPU)."""
    lib = _lib.load()
    cap = lib.gla_fwd_chunked_noalloc_max_scratch()
    assert cap == 64 << 20
    G = 1 << 40  # fake, 16-byte-aligned device addresses: never dereferenced
    P = [FAKE + i * G for i in range(8)]

    def call(B=1, T=64, H=1, dk=64, dv=64, N=1, C=64, ind=_lib.GLA_BF16, cu=None, q=None):
        p = list(P)
        if cu is not None:
            p[5] = cu
        if q is not None:
            p[0] = q
        return lib.gla_fwd_chunked_noalloc(*p, B, T, H, dk, dv, N, C, ind, _lib.GLA_F32, None)

    assert call(B=-1) == _lib.GLA_ERR_INVALID_ARGUMENT
    assert call(q=FAKE + 4) == _lib.GLA_ERR_INVALID_ARGUMENT       # misaligned
    assert call(dk=32) == _lib.GLA_ERR_UNSUPPORTED
    assert call(C=32) == _lib.GLA_ERR_UNSUPPORTED
    assert call(H=0) == _lib.GLA_OK                                # nothing to do
    # one 4M-token sequence over 64 heads: its segment states need far more
    # than the fixed scratch
    need = lib.gla_fwd_chunked_workspace_size(1, 1 << 22, 64, 128, 128, 1, 64, 0, _lib.GLA_BF16)
    assert need > cap
    assert call(T=1 << 22, H=64, dk=128, dv=128) == _lib.GLA_ERR_WORKSPACE
