"""MI355X (gfx950) sink-seeded sliding-window / global attention: Python binding of libmimo_attn.

The binding only marshals arguments to the C ABI (include/mimo_attn.h): it checks tensor
placement, dtype and shape, allocates outputs when none are given, and passes raw device pointers
plus the current HIP stream. Every step of the computation runs in the HIP kernels; there is no
fallback. If the shared library is missing, every call raises.

    o, lse = prefill(q, k, v, window=128, sink=sink)          # q [B, L, Hq, 192] ...
    o, lse = decode(q, k_new, v_new, k_cache, v_cache, cache_len, window=128, ...)
    table = rope_table(n_pos, base=1e4)                        # RoPE (cos, sin), device fp32
    o, lse = prefill(q, k, v, 128, sink=sink, rope=table)      # q, k given before RoPE
    dq, dk, dv, dsink = prefill_backward(q, k, v, o, lse, do, 128, sink=sink)
    cache_append(k_new, v_new, k_cache, v_cache, cache_len, max_len, accept=accepted)
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = ["prefill", "decode", "decode_workspace_size", "prefill_rope_workspace_size", "rope_table", "prefill_backward", "cache_append",
           "backward_workspace_size", "last_error", "version", "library", "LIB_PATH", "MimoError",
           "EXPORTS", "ROPE_DIMS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmimo_attn.so")
EXPORTS = ("mimo_attn_prefill", "mimo_attn_decode", "mimo_attn_decode_workspace_size",
           "mimo_attn_rope_table", "mimo_attn_prefill_rope", "mimo_attn_prefill_rope_workspace_size",
           "mimo_attn_decode_rope", "mimo_attn_decode_noalloc",
           "mimo_attn_prefill_backward", "mimo_attn_prefill_backward_workspace_size",
           "mimo_attn_cache_append",
           "mimo_attn_last_error", "mimo_attn_version")
ROPE_DIMS = 64  # rotated leading Q/K dims

MIMO_F32, MIMO_BF16 = 0, 1
_CODES = {-1: "EINVAL", -2: "EUNSUPPORTED", -3: "EWORKSPACE", -4: "EHIP"}


class MimoError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mimo_attn {_CODES.get(code, code)}: {msg}")
        self.code = code


_lib = None


def library() -> ctypes.CDLL:
    """Loads libmimo_attn.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.mimo_attn_prefill.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp,
                                      f32, vp, vp, vp]
    lib.mimo_attn_prefill.restype = i32
    lib.mimo_attn_decode_workspace_size.argtypes = [i32] * 8
    lib.mimo_attn_decode_workspace_size.restype = sz
    lib.mimo_attn_decode.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp,
                                     vp, i32, i32, vp, vp, f32, i32, vp, sz, vp, vp, vp]
    lib.mimo_attn_decode.restype = i32
    lib.mimo_attn_rope_table.argtypes = [i32, i32, ctypes.c_double, vp, vp]
    lib.mimo_attn_rope_table.restype = i32
    lib.mimo_attn_prefill_rope.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, i32, vp,
                                           vp, f32, vp, i32, i32, vp, sz, vp, vp, vp]
    lib.mimo_attn_prefill_rope.restype = i32
    lib.mimo_attn_prefill_rope_workspace_size.argtypes = [i32] * 6
    lib.mimo_attn_prefill_rope_workspace_size.restype = sz
    lib.mimo_attn_decode_rope.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                          i32, vp, vp, i32, i32, vp, vp, f32, vp, i32, i32, i32, vp,
                                          sz, vp, vp, vp]
    lib.mimo_attn_decode_rope.restype = i32
    lib.mimo_attn_decode_noalloc.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                             i32, vp, vp, i32, i32, vp, vp, f32, i32, vp, vp, vp]
    lib.mimo_attn_decode_noalloc.restype = i32
    lib.mimo_attn_prefill_backward.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                                vp, vp, i32, vp, vp, f32, vp, vp, vp, vp, vp, sz,
                                                vp]
    lib.mimo_attn_prefill_backward.restype = i32
    lib.mimo_attn_prefill_backward_workspace_size.argtypes = [i32, i32, i32]
    lib.mimo_attn_prefill_backward_workspace_size.restype = sz
    lib.mimo_attn_cache_append.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, vp, vp,
                                            vp, i32, vp]
    lib.mimo_attn_cache_append.restype = i32
    lib.mimo_attn_last_error.argtypes = []
    lib.mimo_attn_last_error.restype = ctypes.c_char_p
    lib.mimo_attn_version.argtypes = []
    lib.mimo_attn_version.restype = i32
    _lib = lib
    return lib


def last_error() -> str:
    return library().mimo_attn_last_error().decode()


def version() -> int:
    return library().mimo_attn_version()


def _check(rc: int) -> None:
    if rc != 0:
        raise MimoError(rc, last_error())


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return MIMO_BF16
    if t.dtype == torch.float32:
        return MIMO_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _dev(t, name, dtype=None, ndim=None):
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _kv_map(kv_map, Hq):
    if kv_map is None:
        return None, None
    arr = (ctypes.c_int32 * Hq)(*[int(x) for x in kv_map])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def rope_table(n_pos: int, base: float, out=None, stream=None):
    """(cos, sin) table [n_pos, 32, 2] fp32 of the rotary angles, filled by the library kernel."""
    import torch

    if out is None:
        out = torch.empty((n_pos, ROPE_DIMS // 2, 2), dtype=torch.float32, device="cuda")
    _dev(out, "out", torch.float32, 3)
    if tuple(out.shape) != (n_pos, ROPE_DIMS // 2, 2):
        raise ValueError("out has the wrong shape")
    _check(library().mimo_attn_rope_table(int(n_pos), ROPE_DIMS, float(base), _ptr(out),
                                          _stream(stream)))
    return out


def _rope_arg(rope):
    import torch

    _dev(rope, "rope", torch.float32, 3)
    if tuple(rope.shape[1:]) != (ROPE_DIMS // 2, 2):
        raise ValueError("rope must be a [n_pos, 32, 2] table from rope_table()")
    return rope.shape[0]


def prefill(q, k, v, window: int, sink=None, scale: float | None = None, kv_map=None, out=None,
            lse=None, return_lse: bool = False, stream=None, rope=None, workspace=None,
            rotate_k_once: bool = True):
    """Sink-seeded windowed prefill. q [B, L, Hq, dqk], k [B, L, Hkv, dqk], v [B, L, Hkv, dv].

    window >= L means global causal attention. sink: fp32 [Hq] GPU tensor or None. kv_map: host
    sequence of Hq KV-head indices (None = contiguous groups). rope: None, or a table from
    rope_table() when q and k are given before the rotary embedding; then K is rotated once into a
    workspace (given, or allocated here when the chosen kernel uses one) unless rotate_k_once is
    False, which rotates each K block as it is staged. Returns (o, lse or None).
    """
    import torch

    _dev(q, "q", ndim=4)
    dt = _dtype_code(q)
    _dev(k, "k", q.dtype, 4)
    _dev(v, "v", q.dtype, 4)
    B, L, Hq, dqk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    if tuple(k.shape[:2]) != (B, L) or tuple(v.shape[:3]) != (B, L, Hkv) or k.shape[3] != dqk:
        raise ValueError("q, k, v shapes disagree")
    if sink is not None:
        _dev(sink, "sink", torch.float32, 1)
        if sink.shape[0] != Hq:
            raise ValueError("sink must have Hq entries")
    if out is None:
        out = torch.empty((B, L, Hq, dv), dtype=q.dtype, device=q.device)
    _dev(out, "out", q.dtype, 4)
    if tuple(out.shape) != (B, L, Hq, dv):
        raise ValueError("out has the wrong shape")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, Hq, L):
            raise ValueError("lse has the wrong shape")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    keep, kvm = _kv_map(kv_map, Hq)
    if rope is None:
        rc = library().mimo_attn_prefill(dt, B, L, Hq, Hkv, dqk, dv, _ptr(q), _ptr(k), _ptr(v),
                                         int(window), _ptr(sink), kvm, float(scale), _ptr(out),
                                         _ptr(lse), _stream(stream))
    else:
        n_pos = _rope_arg(rope)
        ws_have = 0
        if not rotate_k_once:
            workspace = None
        elif workspace is None:
            need = prefill_rope_workspace_size(q.dtype, B, L, Hq, Hkv, window)
            if need:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if workspace is not None:
            ws_have = workspace.numel() * workspace.element_size()
        rc = library().mimo_attn_prefill_rope(dt, B, L, Hq, Hkv, dqk, dv, _ptr(q), _ptr(k), _ptr(v),
                                              int(window), _ptr(sink), kvm, float(scale), _ptr(rope),
                                              int(n_pos), ROPE_DIMS, _ptr(workspace), ws_have,
                                              _ptr(out), _ptr(lse), _stream(stream))
    del keep
    _check(rc)
    return out, lse


def prefill_rope_workspace_size(dtype, B: int, L: int, Hq: int, Hkv: int, window: int) -> int:
    """Bytes with which a RoPE prefill rotates K once (0: the chosen kernel has no use for them)."""
    import torch

    code = MIMO_BF16 if dtype in (torch.bfloat16, "bf16") else MIMO_F32
    return int(library().mimo_attn_prefill_rope_workspace_size(code, B, L, Hq, Hkv, int(window)))


def decode_workspace_size(B, T, Hq, Hkv, dv, max_cache_len, window, num_splits=0) -> int:
    return int(library().mimo_attn_decode_workspace_size(B, T, Hq, Hkv, dv, max_cache_len, window,
                                                         num_splits))


def decode(q, k_new, v_new, k_cache, v_cache, cache_len, window: int, max_cache_len: int,
           cache_offset=None, sink=None, scale: float | None = None, kv_map=None,
           num_splits: int = 0, workspace=None, out=None, lse=None, return_lse: bool = False,
           stream=None, rope=None):
    """Decode / MTP verify of T = q.shape[1] new tokens per sequence.

    q [B, T, Hq, dqk]; k_new/v_new [B, T, Hkv, d]; k_cache/v_cache [B, C, Hkv, d];
    cache_len / cache_offset int32 [B] GPU tensors. rope: None, or a table from rope_table() when
    q and k_new are given before the rotary embedding (the cache holds rotated keys). workspace:
    None (allocated here when the split plan needs one), a uint8 tensor, or "static" for
    mimo_attn_decode_noalloc (the library's static scratch; with out, and lse if wanted, given,
    the call allocates nothing). Returns (o, lse or None).
    """
    import torch

    _dev(q, "q", ndim=4)
    dt = _dtype_code(q)
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, q.dtype, 4)
    B, T, Hq, dqk = q.shape
    Hkv, dv, C = k_new.shape[2], v_new.shape[3], k_cache.shape[1]
    if (tuple(k_new.shape) != (B, T, Hkv, dqk) or tuple(v_new.shape[:3]) != (B, T, Hkv)
            or tuple(k_cache.shape) != (B, C, Hkv, dqk) or tuple(v_cache.shape) != (B, C, Hkv, dv)):
        raise ValueError("decode tensor shapes disagree")
    _dev(cache_len, "cache_len", torch.int32, 1)
    if cache_offset is not None:
        _dev(cache_offset, "cache_offset", torch.int32, 1)
    if sink is not None:
        _dev(sink, "sink", torch.float32, 1)
    if out is None:
        out = torch.empty((B, T, Hq, dv), dtype=q.dtype, device=q.device)
    _dev(out, "out", q.dtype, 4)
    if lse is None and return_lse:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, 3)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    keep, kvm = _kv_map(kv_map, Hq)
    if isinstance(workspace, str):  # "static": the library's static scratch, nothing is allocated
        if workspace != "static":
            raise ValueError(f"workspace: a tensor, None or 'static' (got {workspace!r})")
        if rope is not None:
            raise ValueError("the static-scratch decode takes rotated q / k_new (rope=None)")
        rc = library().mimo_attn_decode_noalloc(dt, B, T, Hq, Hkv, dqk, dv, _ptr(q), _ptr(k_new),
                                                _ptr(v_new), _ptr(k_cache), _ptr(v_cache), C,
                                                _ptr(cache_len), _ptr(cache_offset),
                                                int(max_cache_len), int(window), _ptr(sink), kvm,
                                                float(scale), int(num_splits), _ptr(out), _ptr(lse),
                                                _stream(stream))
        del keep
        _check(rc)
        return out, lse
    ws_bytes = decode_workspace_size(B, T, Hq, Hkv, dv, max_cache_len, window, num_splits)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if rope is None:
        rc = library().mimo_attn_decode(dt, B, T, Hq, Hkv, dqk, dv, _ptr(q), _ptr(k_new), _ptr(v_new),
                                        _ptr(k_cache), _ptr(v_cache), C, _ptr(cache_len),
                                        _ptr(cache_offset), int(max_cache_len), int(window),
                                        _ptr(sink), kvm, float(scale), int(num_splits),
                                        _ptr(workspace), ws_have, _ptr(out), _ptr(lse),
                                        _stream(stream))
    else:
        n_pos = _rope_arg(rope)
        rc = library().mimo_attn_decode_rope(dt, B, T, Hq, Hkv, dqk, dv, _ptr(q), _ptr(k_new),
                                             _ptr(v_new), _ptr(k_cache), _ptr(v_cache), C,
                                             _ptr(cache_len), _ptr(cache_offset), int(max_cache_len),
                                             int(window), _ptr(sink), kvm, float(scale), _ptr(rope),
                                             int(n_pos), ROPE_DIMS, int(num_splits), _ptr(workspace),
                                             ws_have, _ptr(out), _ptr(lse), _stream(stream))
    del keep
    _check(rc)
    return out, lse


def backward_workspace_size(B: int, L: int, Hq: int) -> int:
    return int(library().mimo_attn_prefill_backward_workspace_size(B, L, Hq))


def prefill_backward(q, k, v, o, lse, d_o, window: int, sink=None, scale: float | None = None,
                     kv_map=None, want_dsink: bool = True, workspace=None, out=None, stream=None):
    """Gradients of a prefill: returns (dq, dk, dv, dsink or None).

    q, k, v, window, sink, scale, kv_map as passed to prefill(); o and lse are its outputs (lse
    [B, Hq, L] fp32 is required); d_o [B, L, Hq, dv] is the loss gradient of o. out: optional
    (dq, dk, dv) tensors to write. dsink [Hq] fp32 is returned when there is a sink and want_dsink.
    """
    import torch

    _dev(q, "q", ndim=4)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("o", o), ("d_o", d_o)):
        _dev(t, name, q.dtype, 4)
    B, L, Hq, dqk = q.shape
    Hkv, dv_ = k.shape[2], v.shape[3]
    if (tuple(k.shape) != (B, L, Hkv, dqk) or tuple(v.shape) != (B, L, Hkv, dv_)
            or tuple(o.shape) != (B, L, Hq, dv_) or tuple(d_o.shape) != (B, L, Hq, dv_)):
        raise ValueError("q, k, v, o, d_o shapes disagree")
    _dev(lse, "lse", torch.float32, 3)
    if tuple(lse.shape) != (B, Hq, L):
        raise ValueError("lse has the wrong shape")
    if sink is not None:
        _dev(sink, "sink", torch.float32, 1)
        if sink.shape[0] != Hq:
            raise ValueError("sink must have Hq entries")
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _dev(t, name, q.dtype, 4)
        if t.shape != ref.shape:
            raise ValueError(f"{name} has the wrong shape")
    dsink = None
    if sink is not None and want_dsink:
        dsink = torch.empty(Hq, dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    ws_bytes = backward_workspace_size(B, L, Hq)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_have = workspace.numel() * workspace.element_size()
    keep, kvm = _kv_map(kv_map, Hq)
    rc = library().mimo_attn_prefill_backward(dt, B, L, Hq, Hkv, dqk, dv_, _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(o), _ptr(lse), _ptr(d_o), int(window), _ptr(sink),
                                              kvm, float(scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                              _ptr(dsink), _ptr(workspace), ws_have, _stream(stream))
    del keep
    _check(rc)
    return dq, dk, dv, dsink


def cache_append(k_new, v_new, k_cache, v_cache, cache_len, max_cache_len: int, cache_offset=None,
                 accept=None, stream=None):
    """Commit the accepted prefix of a verify step's T new tokens into the cache, in place.

    k_new/v_new [B, T, Hkv, d]; k_cache/v_cache [B, C, Hkv, d]; cache_len int32 [B] (advanced on
    the device); cache_offset, accept: int32 [B] GPU tensors or None (offset 0 / all T accepted).
    Returns cache_len.
    """
    import torch

    _dev(k_new, "k_new", ndim=4)
    dt = _dtype_code(k_new)
    for name, t in (("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, k_new.dtype, 4)
    B, T, Hkv, dqk = k_new.shape
    dv, C = v_new.shape[3], k_cache.shape[1]
    if (tuple(v_new.shape[:3]) != (B, T, Hkv) or tuple(k_cache.shape) != (B, C, Hkv, dqk)
            or tuple(v_cache.shape) != (B, C, Hkv, dv)):
        raise ValueError("cache_append tensor shapes disagree")
    _dev(cache_len, "cache_len", torch.int32, 1)
    for name, t in (("cache_offset", cache_offset), ("accept", accept)):
        if t is not None:
            _dev(t, name, torch.int32, 1)
    _check(library().mimo_attn_cache_append(dt, B, T, Hkv, dqk, dv, _ptr(k_new), _ptr(v_new),
                                            _ptr(k_cache), _ptr(v_cache), C, _ptr(cache_len),
                                            _ptr(cache_offset), _ptr(accept), int(max_cache_len),
                                            _stream(stream)))
    return cache_len
