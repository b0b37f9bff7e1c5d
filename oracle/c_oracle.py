"""ctypes wrapper and build step for the C fp64 oracle (oracle/gla_oracle.c).

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).
``build()`` compiles ``liboracle.so`` next to this file with gcc -O2 -fopenmp.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

__all__ = ["build", "load", "fwd", "bwd", "decode"]


def build(verbose: bool = False) -> str:
    """Compile the C oracle (always recompiles). Returns the library path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o",
           _LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        f = ctypes.POINTER(ctypes.c_float)
        d = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.POINTER(ctypes.c_int64)
        lib.gla_oracle_fwd.argtypes = [f, f, f, f, f, i64] + [ctypes.c_int] * 6 + [d, d, ctypes.c_int]
        lib.gla_oracle_fwd.restype = ctypes.c_int
        lib.gla_oracle_bwd.argtypes = ([f, f, f, f, f, f, f, i64] + [ctypes.c_int] * 6
                                       + [d, d, d, d, d, ctypes.c_int])
        lib.gla_oracle_bwd.restype = ctypes.c_int
        lib.gla_oracle_decode.argtypes = [f, f, f, f, d, d] + [ctypes.c_int] * 5
        lib.gla_oracle_decode.restype = ctypes.c_int
        _lib = lib
    return _lib


def _fp(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def fwd(q, k, v, log_g, S0=None, cu_seqlens=None, nthreads: int = 0):
    """Token-by-token fp64 forward. Same shapes as oracle.gla_oracle.recurrent_forward.

    Returns (o fp64, S_T fp64, threads_used).
    """
    lib = load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    lg = np.ascontiguousarray(log_g, dtype=np.float32)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N = len(cu) - 1
        cu_p = _fp(cu, ctypes.c_int64)
    else:
        cu, N, cu_p = None, B, None
    s0 = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float32)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    ST = np.zeros((N, H, dk, dv), dtype=np.float64)
    used = lib.gla_oracle_fwd(_fp(q, ctypes.c_float), _fp(k, ctypes.c_float),
                              _fp(v, ctypes.c_float), _fp(lg, ctypes.c_float),
                              None if s0 is None else _fp(s0, ctypes.c_float), cu_p,
                              B, T, H, dk, dv, N, _fp(o, ctypes.c_double),
                              _fp(ST, ctypes.c_double), int(nthreads))
    return o, ST, used


def bwd(q, k, v, log_g, dO, dS_T=None, S0=None, cu_seqlens=None, nthreads: int = 0):
    """Token-by-token fp64 backward (the adjoint walk of
    oracle.gla_oracle.recurrent_backward, same shapes and order of results).

    Returns (dq, dk, dv, dlog_g, dS0, threads_used), all fp64.
    """
    lib = load()
    c32 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float32)
    q, k, v, lg, dO = (c32(x) for x in (q, k, v, log_g, dO))
    s0, dst = c32(S0), c32(dS_T)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N = len(cu) - 1
        cu_p = _fp(cu, ctypes.c_int64)
    else:
        cu, N, cu_p = None, B, None
    dq = np.zeros((B, T, H, dk), dtype=np.float64)
    dkk = np.zeros((B, T, H, dk), dtype=np.float64)
    dvv = np.zeros((B, T, H, dv), dtype=np.float64)
    dl = np.zeros((B, T, H), dtype=np.float64)
    dS0 = np.zeros((N, H, dk, dv), dtype=np.float64)
    fp = lambda a: None if a is None else _fp(a, ctypes.c_float)
    used = lib.gla_oracle_bwd(fp(q), fp(k), fp(v), fp(lg), fp(dO), fp(s0), fp(dst), cu_p,
                              B, T, H, dk, dv, N, _fp(dq, ctypes.c_double),
                              _fp(dkk, ctypes.c_double), _fp(dvv, ctypes.c_double),
                              _fp(dl, ctypes.c_double), _fp(dS0, ctypes.c_double), int(nthreads))
    if used < 0:
        raise MemoryError("oracle backward: state buffer allocation failed")
    return dq, dkk, dvv, dl, dS0, used


def decode(q, k, v, log_g, S, nthreads: int = 0):
    """One fp64 decode step. S (fp64 [N,H,dk,dv]) is updated in place.

    Returns (o fp64 [N,H,dv], threads_used).
    """
    lib = load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    lg = np.ascontiguousarray(log_g, dtype=np.float32)
    if S.dtype != np.float64 or not S.flags.c_contiguous:
        raise ValueError("S must be a C-contiguous float64 array (updated in place)")
    N, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((N, H, dv), dtype=np.float64)
    used = lib.gla_oracle_decode(_fp(q, ctypes.c_float), _fp(k, ctypes.c_float),
                                 _fp(v, ctypes.c_float), _fp(lg, ctypes.c_float),
                                 _fp(S, ctypes.c_double), _fp(o, ctypes.c_double),
                                 N, H, dk, dv, int(nthreads))
    return o, used
