"""ctypes loader for libgla.so (the HIP library). Fails loudly if it is missing."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgla.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "gla.h")

GLA_OK = 0
GLA_ERR_INVALID_ARGUMENT = 1
GLA_ERR_UNSUPPORTED = 2
GLA_ERR_WORKSPACE = 3
GLA_ERR_HIP = 4
GLA_F32 = 0
GLA_BF16 = 1

_lib = None


class GLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def load():
    """Load libgla.so once. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libgla.so not found at {LIB_PATH}; build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.gla_status_string.argtypes = [i]
    lib.gla_status_string.restype = ctypes.c_char_p
    lib.gla_fwd_chunked_workspace_size.argtypes = [i] * 9
    lib.gla_fwd_chunked_workspace_size.restype = ctypes.c_size_t
    lib.gla_fwd_chunked.argtypes = [vp] * 8 + [i] * 7 + [i, i, vp, ctypes.c_size_t, vp]
    lib.gla_fwd_chunked.restype = i
    lib.gla_fwd_chunked_noalloc.argtypes = [vp] * 8 + [i] * 7 + [i, i, vp]
    lib.gla_fwd_chunked_noalloc.restype = i
    lib.gla_fwd_chunked_noalloc_max_scratch.argtypes = []
    lib.gla_fwd_chunked_noalloc_max_scratch.restype = ctypes.c_size_t
    lib.gla_fwd_chunked_fixed_decay.argtypes = lib.gla_fwd_chunked.argtypes
    lib.gla_fwd_chunked_fixed_decay.restype = i
    lib.gla_bwd_chunked_workspace_size.argtypes = [i] * 9
    lib.gla_bwd_chunked_workspace_size.restype = ctypes.c_size_t
    lib.gla_bwd_chunked.argtypes = [vp] * 13 + [i] * 7 + [i, vp, ctypes.c_size_t, vp]
    lib.gla_bwd_chunked.restype = i
    lib.gla_decode_step.argtypes = [vp] * 6 + [i] * 4 + [i, i, vp]
    lib.gla_decode_step.restype = i
    lib.gla_decode_step_slots.argtypes = [vp] * 8 + [i] * 5 + [i, i, vp]
    lib.gla_decode_step_slots.restype = i
    lib.gla_mixer_epilogue.argtypes = [vp] * 7 + [ctypes.c_float, vp] + [i] * 4 + [i, i, i, vp]
    lib.gla_mixer_epilogue.restype = i
    lib.gla_decode_slot_order.argtypes = [vp, i, i, ctypes.c_size_t, vp, vp]
    lib.gla_decode_slot_order.restype = i
    lib.gla_decode_mixer.argtypes = ([vp] * 7 + [i] + [vp] * 3 + [ctypes.c_float, vp] + [i] * 4
                                     + [i, i, vp])
    lib.gla_decode_mixer.restype = i
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gla_status_string(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != GLA_OK:
        raise GLAError(status, what)
