"""gla_fwd_chunked_noalloc, called through the C ABI, against gla_fwd_chunked
with a caller-allocated workspace: the same kernels and the same plan, so the
outputs must agree bit for bit; both are also held to the oracle's bar.

Two calls in a row on one GPU, the second with a smaller input (a packed
batch), both split into segments so that both use the library's scratch;
the second call must not see anything of the first one's scratch contents.
"""
import ctypes

import numpy as np
import pytest

import gpu_util as gu
from gated_linear_attention_amd import _lib, synth
from oracle import c_oracle

pytestmark = pytest.mark.gpu


def _abi_forward(lib, q, k, v, g, S0, cu, C, noalloc):
    """One forward through the C ABI (ctypes; torch only supplies memory and
    the stream). Returns (o, S_T) as device tensors."""
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = B if cu is None else cu.numel() - 1
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=q.device)
    ST = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    ind = _lib.GLA_BF16 if q.dtype == torch.bfloat16 else _lib.GLA_F32
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    args = [p(q), p(k), p(v), p(g), p(S0), p(cu), p(o), p(ST), B, T, H, dk, dv, N, C, ind,
            _lib.GLA_F32]
    if noalloc:
        st = lib.gla_fwd_chunked_noalloc(*args, stream)
    else:
        nb = lib.gla_fwd_chunked_workspace_size(B, T, H, dk, dv, N, C, int(cu is not None), ind)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=q.device)
        st = lib.gla_fwd_chunked(*args, p(ws), nb, stream)
    assert st == _lib.GLA_OK, _lib.status_string(st)
    return o, ST


def _case(lib, w, lengths, C):
    import torch
    q, k, v, lg, S0, cu = synth.make_forward_inputs(w, lengths=lengths)
    td = gu.in_dtype(w.dtype)
    d = lambda x, t=None: gu.dev(x, t)
    qd, kd, vd, gd, S0d, cud = d(q, td), d(k, td), d(v, td), d(lg), d(S0), d(cu)
    N = q.shape[0] if cu is None else len(cu) - 1
    need = lib.gla_fwd_chunked_workspace_size(q.shape[0], q.shape[1], q.shape[2], w.dk, w.dv, N,
                                              C, int(cu is not None),
                                              _lib.GLA_BF16 if w.dtype == "bf16" else _lib.GLA_F32)
    assert 0 < need <= lib.gla_fwd_chunked_noalloc_max_scratch(), need
    o1, S1 = _abi_forward(lib, qd, kd, vd, gd, S0d, cud, C, noalloc=True)
    o2, S2 = _abi_forward(lib, qd, kd, vd, gd, S0d, cud, C, noalloc=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    o_ref, S_ref, _ = c_oracle.fwd(q, k, v, lg, S0, cu, nthreads=16)
    eo, eS = gu.tok_error(gu.host(o1), o_ref, cu), gu.state_error(gu.host(S1), S_ref)
    tol = gu.TOL_BF16 if w.dtype == "bf16" else gu.TOL_F32
    gu.say(f"   scratch {need} B; o err {eo:.2e}  S_T err {eS:.2e}; bit-identical to the "
           f"workspace call")
    assert eo <= tol and eS <= tol, (eo, eS)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_two_calls_second_smaller(dtype, monkeypatch):
    gu.say(f"no-alloc forward, two calls, {dtype}")
    lib = _lib.load()
    monkeypatch.setenv("GLA_SEG_LEN", "256")
    w = synth.Workload("n", B=2, T=1500, H=3, dk=128, dv=128, dtype=dtype, gate_bias=3.0,
                       s0_std=0.02, chunk=64, seed=90)
    _case(lib, w, None, 64)                       # dense, 2 x 1,500 tokens
    _case(lib, w, [700, 0, 37, 300], 64)          # packed, 1,037 tokens
