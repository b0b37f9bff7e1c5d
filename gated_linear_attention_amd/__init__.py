"""Gated linear attention (GLA) for AMD MI355X: Python binding of libgla.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libgla.so (see include/gla.h for the C ABI). PyTorch supplies
device memory and the current HIP stream.

    o, S_T = fwd_chunked(q, k, v, g, S0=None, cu_seqlens=None, chunk_size=64)
    o, S_T = fwd_chunked_fixed_decay(q, k, v, log_lambda, S0=None, cu_seqlens=None)
    o, S_T = fwd_chunked_noalloc(q, k, v, g, S0=None, cu_seqlens=None)  # no workspace
    dq, dk, dv, dg, dS0 = bwd_chunked(q, k, v, g, dO, S0=None, cu_seqlens=None, dS_T=None)
    o = decode_step(q, k, v, g, S)          # S updated in place
    order = slot_order(slots, P, H * dk * dv * 4)  # once per step: the pool's streaming order
    o = decode_step_slots(q, k, v, g, S_pool, slots, order=order)   # S_pool[slots] in place
    z = mixer_epilogue(o, q, k, v, g_out, a, rms_w, eps)  # self-augmentation, RMSNorm, SiLU gate
    z = decode_mixer(q, k, v, g, S, g_out, a, rms_w, eps, slots=None, order=None)  # fused

Shapes follow the C ABI: q, k [B, T, H, dk]; v [B, T, H, dv]; g [B, T, H]
fp32 natural-log gates; S0 / S_T [N, H, dk, dv] fp32; cu_seqlens int32 [N+1]
on the device (packed batch, B == 1).
"""
from __future__ import annotations

from . import _lib
from ._lib import GLAError, GLA_BF16, GLA_F32

__all__ = ["fwd_chunked", "fwd_chunked_fixed_decay", "fwd_chunked_noalloc", "bwd_chunked",
           "decode_step",
           "decode_step_slots", "slot_order", "mixer_epilogue", "decode_mixer",
           "head_rms_weights",
           "workspace_size",
           "GLAError", "library_path"]


def library_path() -> str:
    return _lib.LIB_PATH


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t == torch.bfloat16:
        return GLA_BF16
    if t == torch.float32:
        return GLA_F32
    raise TypeError(f"unsupported dtype {t}; expected torch.bfloat16 or torch.float32")


def _ptr(x):
    return None if x is None else x.data_ptr()


def _require(x, name, dtype=None, device=None, align=16):
    """Contiguous, of the given dtype and device, and starting on an `align`-byte
    boundary (16 for tensors; 4 for the log-gate streams and int32 arrays)."""
    if x is None:
        return
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be in GPU memory, got a {x.device.type} tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if x.data_ptr() % align:
        raise ValueError(f"{name} must start on a {align}-byte boundary (a view with a storage "
                         f"offset may not); pass a copy")
    if dtype is not None and x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {x.dtype}")
    if device is not None and x.device != device:
        raise ValueError(f"{name} must be on {device}, got {x.device}")


def workspace_size(B, T, H, dk, dv, num_seqs, chunk_size=64, has_cu_seqlens=False,
                   in_dtype=None) -> int:
    torch = _torch()
    code = _dtype_code(torch.bfloat16 if in_dtype is None else in_dtype)
    return int(_lib.load().gla_fwd_chunked_workspace_size(
        B, T, H, dk, dv, num_seqs, chunk_size, int(bool(has_cu_seqlens)), code))


def fwd_chunked(q, k, v, g, S0=None, cu_seqlens=None, chunk_size: int = 64, out_dtype=None,
                output_final_state: bool = True, o=None, S_T=None, workspace=None):
    """Chunked GLA forward. Returns (o, S_T) (S_T is None if not requested)."""
    return _fwd(q, k, v, g, S0, cu_seqlens, chunk_size, out_dtype, output_final_state, o, S_T,
                workspace, fixed_decay=False)


def fwd_chunked_fixed_decay(q, k, v, log_lambda, S0=None, cu_seqlens=None, chunk_size: int = 64,
                            out_dtype=None, output_final_state: bool = True, o=None, S_T=None,
                            workspace=None):
    """Chunked GLA forward with one fixed log-decay per head (log_lambda [H]
    fp32): no per-token gate stream. Returns (o, S_T)."""
    return _fwd(q, k, v, log_lambda, S0, cu_seqlens, chunk_size, out_dtype, output_final_state,
                o, S_T, workspace, fixed_decay=True)


def fwd_chunked_noalloc(q, k, v, g, S0=None, cu_seqlens=None, chunk_size: int = 64,
                        out_dtype=None, output_final_state: bool = True, o=None, S_T=None):
    """fwd_chunked through gla_fwd_chunked_noalloc: the library's fixed per-GPU
    scratch instead of a workspace (nothing is allocated for it; pass o and
    S_T to allocate nothing at all). Returns (o, S_T)."""
    return _fwd(q, k, v, g, S0, cu_seqlens, chunk_size, out_dtype, output_final_state, o, S_T,
                None, fixed_decay=False, noalloc=True)


def _fwd(q, k, v, g, S0, cu_seqlens, chunk_size, out_dtype, output_final_state, o, S_T,
         workspace, fixed_decay, noalloc=False):
    torch = _torch()
    lib = _lib.load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or g.dim() != (1 if fixed_decay else 3):
        raise ValueError("expected q, k, v [B, T, H, d] and "
                         + ("log_lambda [H]" if fixed_decay else "g [B, T, H]"))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _require(q, "q", None, dev)
    _require(k, "k", q.dtype, dev)
    _require(v, "v", q.dtype, dev)
    _require(g, "g", torch.float32, dev, align=4)
    _require(S0, "S0", torch.float32, dev)
    _require(cu_seqlens, "cu_seqlens", torch.int32, dev, align=4)
    g_shape = (H,) if fixed_decay else (B, T, H)
    if tuple(k.shape) != (B, T, H, dk) or tuple(v.shape[:3]) != (B, T, H) or tuple(g.shape) != g_shape:
        raise ValueError("inconsistent q/k/v/g shapes")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if S0 is not None and tuple(S0.shape) != (N, H, dk, dv):
        raise ValueError(f"S0 must be [{N}, {H}, {dk}, {dv}]")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    _require(o, "o", out_dtype, dev)
    if output_final_state and S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    _require(S_T, "S_T", torch.float32, dev)
    in_code = _dtype_code(q.dtype)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if noalloc:
        st = lib.gla_fwd_chunked_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S0),
                                         _ptr(cu_seqlens), _ptr(o), _ptr(S_T), B, T, H, dk, dv,
                                         N, chunk_size, in_code, _dtype_code(out_dtype), stream)
        _lib.check(st, "gla_fwd_chunked_noalloc")
        return o, S_T
    ws_bytes = int(lib.gla_fwd_chunked_workspace_size(B, T, H, dk, dv, N, chunk_size,
                                                      int(cu_seqlens is not None), in_code))
    if ws_bytes > 0 and (workspace is None or workspace.numel() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fn = lib.gla_fwd_chunked_fixed_decay if fixed_decay else lib.gla_fwd_chunked
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S0), _ptr(cu_seqlens), _ptr(o), _ptr(S_T),
            B, T, H, dk, dv, N, chunk_size, in_code, _dtype_code(out_dtype),
            _ptr(workspace) if ws_bytes > 0 else None, ws_bytes, stream)
    _lib.check(st, "gla_fwd_chunked_fixed_decay" if fixed_decay else "gla_fwd_chunked")
    return o, S_T


def bwd_chunked(q, k, v, g, dO, S0=None, cu_seqlens=None, dS_T=None, chunk_size: int = 64,
                need_dS0: bool = True, workspace=None):
    """Backward of fwd_chunked for upstream gradients dO (and dS_T of the final
    state, None for zero). Returns fp32 (dq, dk, dv, dg, dS0); dS0 is None when
    not requested."""
    torch = _torch()
    lib = _lib.load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or g.dim() != 3 or dO.dim() != 4:
        raise ValueError("expected q, k [B, T, H, dk], v, dO [B, T, H, dv] and g [B, T, H]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _require(q, "q", None, dev)
    _require(k, "k", q.dtype, dev)
    _require(v, "v", q.dtype, dev)
    _require(dO, "dO", q.dtype, dev)
    _require(g, "g", torch.float32, dev, align=4)
    _require(S0, "S0", torch.float32, dev)
    _require(dS_T, "dS_T", torch.float32, dev)
    _require(cu_seqlens, "cu_seqlens", torch.int32, dev, align=4)
    if (tuple(k.shape) != (B, T, H, dk) or tuple(v.shape[:3]) != (B, T, H)
            or tuple(g.shape) != (B, T, H) or tuple(dO.shape) != tuple(v.shape)):
        raise ValueError("inconsistent q/k/v/g/dO shapes")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    for name, x in (("S0", S0), ("dS_T", dS_T)):
        if x is not None and tuple(x.shape) != (N, H, dk, dv):
            raise ValueError(f"{name} must be [{N}, {H}, {dk}, {dv}]")
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty((B, T, H, dk), **f32)
    dkk = torch.empty((B, T, H, dk), **f32)
    dvv = torch.empty((B, T, H, dv), **f32)
    dg = torch.empty((B, T, H), **f32)
    dS0 = torch.empty((N, H, dk, dv), **f32) if need_dS0 else None
    in_code = _dtype_code(q.dtype)
    ws_bytes = int(lib.gla_bwd_chunked_workspace_size(B, T, H, dk, dv, N, chunk_size,
                                                      int(cu_seqlens is not None), in_code))
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.gla_bwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S0), _ptr(cu_seqlens),
                             _ptr(dO), _ptr(dS_T), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg),
                             _ptr(dS0), B, T, H, dk, dv, N, chunk_size, in_code,
                             _ptr(workspace), ws_bytes, stream)
    _lib.check(st, "gla_bwd_chunked")
    return dq, dkk, dvv, dg, dS0


def decode_step(q, k, v, g, S, out_dtype=None, o=None):
    """One recurrent decode step; S [N, H, dk, dv] fp32 is updated in place. Returns o."""
    torch = _torch()
    lib = _lib.load()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or g.dim() != 2 or S.dim() != 4:
        raise ValueError("expected q, k [N, H, dk], v [N, H, dv], g [N, H], S [N, H, dk, dv]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _require(q, "q", None, dev)
    _require(k, "k", q.dtype, dev)
    _require(v, "v", q.dtype, dev)
    _require(g, "g", torch.float32, dev, align=4)
    _require(S, "S", torch.float32, dev)
    if tuple(S.shape) != (N, H, dk, dv) or tuple(g.shape) != (N, H):
        raise ValueError("inconsistent decode shapes")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    _require(o, "o", out_dtype, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.gla_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S), _ptr(o), N, H, dk, dv,
                             _dtype_code(q.dtype), _dtype_code(out_dtype), stream)
    _lib.check(st, "gla_decode_step")
    return o


def slot_order(slots, P, slot_bytes=0):
    """The streaming order (int32 [2, N] on the device: the requests in pool
    order, padded lanes last, then their slots) of a serving batch whose
    requests use pool entries slots (int32 [N]) of a P-entry pool whose
    entries are slot_bytes each (H * dk * dv * 4; 0 for plain slot order):
    computed on the GPU, once per step, and passed to every layer's
    decode_step_slots / decode_mixer."""
    torch = _torch()
    lib = _lib.load()
    _require(slots, "slots", torch.int32, slots.device, align=4)
    if slot_bytes < 0:
        raise ValueError("slot_bytes must be >= 0")
    N = slots.numel()
    order = torch.empty((2, N), dtype=torch.int32, device=slots.device)
    stream = torch.cuda.current_stream(slots.device).cuda_stream
    st = lib.gla_decode_slot_order(_ptr(slots), N, int(P), int(slot_bytes), _ptr(order), stream)
    _lib.check(st, "gla_decode_slot_order")
    return order


def decode_step_slots(q, k, v, g, S_pool, slots, out_dtype=None, o=None, order=None):
    """Decode step over a pool of states: request n reads and updates
    S_pool[slots[n]] ([P, H, dk, dv] fp32, in place); slots (int32 [N], on the
    device) outside [0, P) mark padded lanes (no state touched, o = 0). order
    (int32 [2, N], from slot_order) sets the streaming order only. Returns o."""
    torch = _torch()
    lib = _lib.load()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or g.dim() != 2 or S_pool.dim() != 4:
        raise ValueError("expected q, k [N, H, dk], v [N, H, dv], g [N, H], S_pool [P, H, dk, dv]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    P = S_pool.shape[0]
    dev = q.device
    _require(q, "q", None, dev)
    _require(k, "k", q.dtype, dev)
    _require(v, "v", q.dtype, dev)
    _require(g, "g", torch.float32, dev, align=4)
    _require(S_pool, "S_pool", torch.float32, dev)
    _require(slots, "slots", torch.int32, dev, align=4)
    _require(order, "order", torch.int32, dev, align=4)
    if (tuple(S_pool.shape[1:]) != (H, dk, dv) or tuple(g.shape) != (N, H) or slots.numel() != N
            or (order is not None and tuple(order.shape) != (2, N))):
        raise ValueError("inconsistent decode shapes")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    _require(o, "o", out_dtype, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.gla_decode_step_slots(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S_pool), _ptr(slots),
                                   _ptr(order), _ptr(o), N, P, H, dk, dv, _dtype_code(q.dtype),
                                   _dtype_code(out_dtype), stream)
    _lib.check(st, "gla_decode_step_slots")
    return o


def head_rms_weights(tier_weights, tier):
    """Per-head RMSNorm weights [H, dv] from one weight row per decay tier
    ([n_tiers, dv]) and each head's tier ([H] int): the heads of a tier share
    their row (a gather of parameters, done once per model)."""
    torch = _torch()
    return tier_weights.index_select(0, tier.to(torch.long)).contiguous()


def mixer_epilogue(o, q, k, v, g, a, rms_w, eps: float = 1e-6, out_dtype=None, z=None):
    """Token-mixer epilogue: z = RMSNorm_h(o + sigmoid(q.(a*k)) v) * silu(g).

    o, v, g [..., H, dv]; q, k [..., H, dk] (q, k, v, g one dtype); a [H, dk]
    and rms_w [H, dv] fp32 (head_rms_weights builds rms_w from tier rows).
    z may be o (in place) when out_dtype is o's dtype; out_dtype defaults to
    z's dtype when z is given, else to o's. Returns z."""
    torch = _torch()
    lib = _lib.load()
    H, dv = o.shape[-2], o.shape[-1]
    dk = q.shape[-1]
    dev = o.device
    lead = tuple(o.shape[:-2])
    n_tok = 1
    for x in lead:
        n_tok *= int(x)
    _require(o, "o", None, dev)
    _require(q, "q", None, dev)
    _require(k, "k", q.dtype, dev)
    _require(v, "v", q.dtype, dev)
    _require(g, "g", q.dtype, dev)
    _require(a, "a", torch.float32, dev)
    _require(rms_w, "rms_w", torch.float32, dev)
    if (tuple(q.shape) != lead + (H, dk) or tuple(k.shape) != lead + (H, dk)
            or tuple(v.shape) != lead + (H, dv) or tuple(g.shape) != lead + (H, dv)
            or tuple(a.shape) != (H, dk) or tuple(rms_w.shape) != (H, dv)):
        raise ValueError("inconsistent o/q/k/v/g/a/rms_w shapes")
    if out_dtype is None:
        out_dtype = o.dtype if z is None else z.dtype
    if z is None:
        z = torch.empty(lead + (H, dv), dtype=out_dtype, device=dev)
    _require(z, "z", out_dtype, dev)
    if tuple(z.shape) != lead + (H, dv):
        raise ValueError("z has the wrong shape")
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.gla_mixer_epilogue(_ptr(o), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(a),
                                _ptr(rms_w), float(eps), _ptr(z), n_tok, H, dk, dv,
                                _dtype_code(o.dtype), _dtype_code(q.dtype),
                                _dtype_code(out_dtype), stream)
    _lib.check(st, "gla_mixer_epilogue")
    return z


def decode_mixer(q, k, v, g, S, g_out, a, rms_w, eps: float = 1e-6, slots=None,
                 out_dtype=None, z=None, order=None):
    """One decode step with the mixer epilogue fused: S (dense [N, H, dk, dv],
    or a pool [P, H, dk, dv] addressed by int32 slots [N], streamed in the
    optional order from slot_order) is updated in place and z = epilogue(o)
    is returned; o itself is not materialised."""
    torch = _torch()
    lib = _lib.load()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or g.dim() != 2 or S.dim() != 4:
        raise ValueError("expected q, k [N, H, dk], v [N, H, dv], g [N, H], S [., H, dk, dv]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    for x, name, dt in ((q, "q", None), (k, "k", q.dtype), (v, "v", q.dtype),
                        (S, "S", torch.float32), (g_out, "g_out", q.dtype),
                        (a, "a", torch.float32), (rms_w, "rms_w", torch.float32)):
        _require(x, name, dt, dev)
    _require(g, "g", torch.float32, dev, align=4)
    _require(slots, "slots", torch.int32, dev, align=4)
    _require(order, "order", torch.int32, dev, align=4)
    if order is not None and (slots is None or tuple(order.shape) != (2, N)):
        raise ValueError("order needs slots and one entry per request")
    if (tuple(S.shape[1:]) != (H, dk, dv) or tuple(g.shape) != (N, H)
            or tuple(g_out.shape) != (N, H, dv) or tuple(a.shape) != (H, dk)
            or tuple(rms_w.shape) != (H, dv) or (slots is None and S.shape[0] != N)
            or (slots is not None and slots.numel() != N)):
        raise ValueError("inconsistent decode_mixer shapes")
    if out_dtype is None:
        out_dtype = torch.float32 if z is None else z.dtype
    if z is None:
        z = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    _require(z, "z", out_dtype, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.gla_decode_mixer(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S), _ptr(slots),
                              _ptr(order), S.shape[0], _ptr(g_out), _ptr(a), _ptr(rms_w), float(eps), _ptr(z),
                              N, H, dk, dv, _dtype_code(q.dtype), _dtype_code(out_dtype), stream)
    _lib.check(st, "gla_decode_mixer")
    return z

