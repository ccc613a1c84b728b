"""ctypes binding for ``librelattn.so`` (the C ABI declared in include/relattn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch supplies device memory (``torch.empty`` for
outputs and the decode workspace) and the stream (the caller's current
stream).  There is no CPU or eager fallback: if the library cannot be loaded,
or a call returns an error, a ``RelAttnError`` is raised.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

__all__ = ["RelAttnError", "library_path", "load_library", "prefill", "extend", "decode", "decode_noalloc",
           "decode_paged", "decode_plan",
           "rel_logits", "scale_factor", "version"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "librelattn.so"

RA_BF16 = 1
RA_F32 = 2
_DTYPE_CODE = {torch.bfloat16: RA_BF16, torch.float32: RA_F32}


class RelAttnError(RuntimeError):
    """A non-zero return from the library, with its message."""


def library_path() -> str:
    return os.environ.get("RELATTN_LIBRARY", os.path.join(_HERE, _LIB_NAME))


_lib = None
_lock = threading.Lock()


def _declare(lib):
    c = ctypes
    vp, i32, i64, f32, sz = c.c_void_p, c.c_int, c.c_longlong, c.c_float, c.c_size_t
    lib.rel_attn_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                     f32, i32, i32, i32, vp]
    lib.rel_attn_prefill.restype = i32
    lib.rel_attn_extend.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, i32, vp, i32, i32,
                                    i32, i32, i32, i32, i32, f32, i32, i32, i32, vp]
    lib.rel_attn_extend.restype = i32
    lib.rel_attn_extend_mx.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, i32, vp, i32, i32,
                                       i32, i32, i32, i32, i32, f32, i32, i32, i32, vp]
    lib.rel_attn_extend_mx.restype = i32
    lib.rel_attn_decode_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32,
                                         c.POINTER(i32), c.POINTER(sz)]
    lib.rel_attn_decode_plan.restype = i32
    lib.rel_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    f32, i32, i32, i32, i32, vp, sz, vp]
    lib.rel_attn_decode.restype = i32
    lib.rel_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                            f32, i32, i32, i32, i32, vp]
    lib.rel_attn_decode_noalloc.restype = i32
    lib.rel_attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, i32, i32, i32,
                                          i32, i32, i32, i32, f32, i32, i32, i32, i32, vp, sz, vp]
    lib.rel_attn_decode_paged.restype = i32
    lib.rel_attn_prologue.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp,
                                      i32, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.rel_attn_prologue.restype = i32
    lib.rel_attn_prologue_mx.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp,
                                         vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.rel_attn_prologue_mx.restype = i32
    lib.rel_attn_decode_mx.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, i32,
                                       i32, i32, f32, i32, i32, i32, i32, vp, sz, vp]
    lib.rel_attn_decode_mx.restype = i32
    lib.rel_attn_backward_plan.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_int),
                                           ctypes.POINTER(ctypes.c_size_t)]
    lib.rel_attn_backward_plan.restype = i32
    lib.rel_attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                      i32, f32, i32, i32, i32, i32, vp, ctypes.c_size_t, vp]
    lib.rel_attn_backward.restype = i32
    lib.rel_mx_quantize.argtypes = [vp, vp, vp, i32, i64, i32, vp]
    lib.rel_mx_quantize.restype = i32
    lib.rel_logits.argtypes = [vp, vp, vp, i32, i64, i32, i32, i32, i32, i64, vp]
    lib.rel_logits.restype = i32
    lib.rel_attn_last_error.argtypes = []
    lib.rel_attn_last_error.restype = c.c_char_p
    lib.rel_attn_version.argtypes = []
    lib.rel_attn_version.restype = i32
    lib.rel_attn_scale_factor.argtypes = [i32, i64]
    lib.rel_attn_scale_factor.restype = c.c_double
    return lib


def load_library():
    """Load (once) and return the ctypes handle; raise if the library is missing."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise RelAttnError(
                    f"{path} not found: build the HIP library first "
                    "(python -m transformer_attention_query_amd.build)")
            _lib = _declare(ctypes.CDLL(path))
    return _lib


def _check(rc: int):
    if rc != 0:
        msg = load_library().rel_attn_last_error()
        raise RelAttnError(f"relattn error {rc}: {msg.decode() if msg else ''}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, device: torch.device, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def version() -> int:
    return load_library().rel_attn_version()


def scale_factor(seq_len: int, log_scale: bool) -> float:
    """The library's length-dependent log-scale s for a sequence of ``seq_len`` tokens."""
    return float(load_library().rel_attn_scale_factor(1 if log_scale else 0, int(seq_len)))


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, r: Optional[torch.Tensor],
            P_cols: Optional[torch.Tensor], alpha: float, rel_extent: int, window: int = 0,
            log_scale: bool = False, return_lse: bool = True,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None
            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Relative-attention prefill on the current stream.

    q [B,T,Hq,D], k/v [B,T,Hkv,D], r [B,T,Hq,d_r], P_cols [E,d_r] (row d = the
    projection vector of distance d), all of one dtype (bf16 or fp32) on one GPU.
    Returns out [B,T,Hq,D] (input dtype) and lse [B,Hq,T] fp32 (or None).
    """
    lib = load_library()
    dev = q.device
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    _need(q, "q", dt, dev, 4)
    _need(k, "k", dt, dev, 4)
    _need(v, "v", dt, dev, 4)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, T, Hkv, D) or v.shape != k.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} does not match q {tuple(q.shape)}")
    d_r = 0
    if rel_extent > 0:
        _need(r, "r", dt, dev, 4)
        _need(P_cols, "P_cols", dt, dev, 2)
        d_r = r.shape[3]
        if r.shape[:3] != (B, T, Hq):
            raise ValueError(f"r shape {tuple(r.shape)} does not match q")
        if P_cols.shape != (rel_extent, d_r):
            raise ValueError(f"P_cols must be [rel_extent={rel_extent}, d_r={d_r}], got {tuple(P_cols.shape)}")
    else:
        r = None
        P_cols = None
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", dt, dev, 4)
    if return_lse and lse is None:
        lse = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
    elif not return_lse:
        lse = None
    _check(lib.rel_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(r), _ptr(P_cols), _ptr(out), _ptr(lse),
                                _DTYPE_CODE[dt], B, T, Hq, Hkv, D, d_r, float(alpha), int(rel_extent),
                                int(window), 1 if log_scale else 0, _stream(dev)))
    return out, lse


def extend(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, r: Optional[torch.Tensor],
           P_cols: Optional[torch.Tensor], alpha: float, rel_extent: int, window: int,
           log_scale: bool, q_start: torch.Tensor, kv_len: torch.Tensor, max_q: int,
           block_table: Optional[torch.Tensor] = None, return_lse: bool = True,
           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None
           ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """New rows of packed sequences against their KV caches (rel_attn_extend).

    q [total_q,Hq,D], r [total_q,Hq,d_r] packed by ``q_start`` [B+1] (int32,
    device); ``kv_len`` [B] (int32, device) cached tokens per sequence, the
    last q_start[b+1]-q_start[b] of which are the new rows; ``max_q`` a host
    bound on the new rows of any sequence.  k/v: contiguous caches
    [B,cache_len,Hkv,D], or with ``block_table`` [B,max_pages] (int32, device)
    paged caches [num_pages,page_size,Hkv,D].  Returns out [total_q,Hq,D] and
    lse [Hq,total_q] fp32 (or None).
    """
    lib = load_library()
    dev = q.device
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    _need(q, "q", dt, dev, 3)
    _need(k, "k", dt, dev, 4)
    _need(v, "v", dt, dev, 4)
    _need(q_start, "q_start", torch.int32, dev, 1)
    _need(kv_len, "kv_len", torch.int32, dev, 1)
    total_q, Hq, D = q.shape
    B = kv_len.shape[0]
    if q_start.shape[0] != B + 1:
        raise ValueError(f"q_start must have B+1 = {B + 1} entries, got {q_start.shape[0]}")
    if v.shape != k.shape:
        raise ValueError(f"v shape {tuple(v.shape)} differs from k {tuple(k.shape)}")
    Hkv = k.shape[2]
    if block_table is None:
        cache_len, max_pages, num_pages, page_size = k.shape[1], 0, 0, 0
        if k.shape[0] != B:
            raise ValueError(f"contiguous caches must be [B={B}, cache_len, Hkv, D], got {tuple(k.shape)}")
    else:
        _need(block_table, "block_table", torch.int32, dev, 2)
        if block_table.shape[0] != B:
            raise ValueError(f"block_table must be [B={B}, max_pages], got {tuple(block_table.shape)}")
        cache_len, max_pages, num_pages, page_size = 0, block_table.shape[1], k.shape[0], k.shape[1]
    d_r = 0
    if rel_extent > 0:
        _need(r, "r", dt, dev, 3)
        _need(P_cols, "P_cols", dt, dev, 2)
        d_r = r.shape[2]
        if r.shape[:2] != (total_q, Hq):
            raise ValueError(f"r shape {tuple(r.shape)} does not match q")
        if P_cols.shape != (rel_extent, d_r):
            raise ValueError(f"P_cols must be [rel_extent={rel_extent}, d_r={d_r}], got {tuple(P_cols.shape)}")
    else:
        r = None
        P_cols = None
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", dt, dev, 3)
    if return_lse and lse is None:
        lse = torch.empty(Hq, total_q, dtype=torch.float32, device=dev)
    elif not return_lse:
        lse = None
    _check(lib.rel_attn_extend(_ptr(q), _ptr(k), _ptr(v), _ptr(r), _ptr(P_cols), _ptr(out), _ptr(lse),
                               _DTYPE_CODE[dt], B, total_q, int(max_q), _ptr(q_start), _ptr(kv_len),
                               cache_len, _ptr(block_table), max_pages, num_pages, page_size,
                               Hq, Hkv, D, d_r, float(alpha), int(rel_extent), int(window),
                               1 if log_scale else 0, _stream(dev)))
    return out, lse


def extend_mx(q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, v_codes: torch.Tensor,
              v_scales: torch.Tensor, r: Optional[torch.Tensor], P_cols: Optional[torch.Tensor], alpha: float,
              rel_extent: int, window: int, log_scale: bool, q_start: torch.Tensor, kv_len: torch.Tensor,
              max_q: int, block_table: Optional[torch.Tensor] = None, return_lse: bool = True
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``extend`` over MXFP8 caches (rel_attn_extend_mx): codes [.., Hkv, D]
    and scales [.., Hkv, D/32] (uint8) as ``mx_quantize`` / ``prologue_mx``
    write them, contiguous [B,cache_len,..] or paged [num_pages,page_size,..]
    with ``block_table``.  q, r, P_cols bf16.  Returns out [total_q,Hq,D] bf16
    and lse [Hq,total_q] fp32 (or None)."""
    lib = load_library()
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    for name, t in (("k_codes", k_codes), ("v_codes", v_codes), ("k_scales", k_scales), ("v_scales", v_scales)):
        _need(t, name, torch.uint8, dev, 4)
    _need(q_start, "q_start", torch.int32, dev, 1)
    _need(kv_len, "kv_len", torch.int32, dev, 1)
    total_q, Hq, D = q.shape
    B = kv_len.shape[0]
    if q_start.shape[0] != B + 1:
        raise ValueError(f"q_start must have B+1 = {B + 1} entries, got {q_start.shape[0]}")
    if v_codes.shape != k_codes.shape or k_scales.shape != k_codes.shape[:3] + (D // 32,) or \
            v_scales.shape != k_scales.shape:
        raise ValueError("code and scale shapes do not match")
    Hkv = k_codes.shape[2]
    if block_table is None:
        cache_len, max_pages, num_pages, page_size = k_codes.shape[1], 0, 0, 0
        if k_codes.shape[0] != B:
            raise ValueError(f"contiguous caches must be [B={B}, cache_len, Hkv, D], got {tuple(k_codes.shape)}")
    else:
        _need(block_table, "block_table", torch.int32, dev, 2)
        if block_table.shape[0] != B:
            raise ValueError(f"block_table must be [B={B}, max_pages], got {tuple(block_table.shape)}")
        cache_len, max_pages, num_pages, page_size = 0, block_table.shape[1], k_codes.shape[0], k_codes.shape[1]
    d_r = 0
    if rel_extent > 0:
        _need(r, "r", torch.bfloat16, dev, 3)
        _need(P_cols, "P_cols", torch.bfloat16, dev, 2)
        d_r = r.shape[2]
        if r.shape[:2] != (total_q, Hq):
            raise ValueError(f"r shape {tuple(r.shape)} does not match q")
        if P_cols.shape != (rel_extent, d_r):
            raise ValueError(f"P_cols must be [rel_extent={rel_extent}, d_r={d_r}], got {tuple(P_cols.shape)}")
    else:
        r = None
        P_cols = None
    out = torch.empty_like(q)
    lse = torch.empty(Hq, total_q, dtype=torch.float32, device=dev) if return_lse else None
    _check(lib.rel_attn_extend_mx(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales), _ptr(r),
                                  _ptr(P_cols), _ptr(out), _ptr(lse), B, total_q, int(max_q), _ptr(q_start),
                                  _ptr(kv_len), cache_len, _ptr(block_table), max_pages, num_pages, page_size,
                                  Hq, Hkv, D, d_r, float(alpha), int(rel_extent), int(window),
                                  1 if log_scale else 0, _stream(dev)))
    return out, lse


def decode_plan(B: int, L: int, Hq: int, Hkv: int, D: int = 128, num_splits: int = 0,
                window: int = 0, rel_extent: int = 0) -> Tuple[int, int]:
    """(num_splits, workspace_bytes) the decode call will use; a pure function of the shape."""
    lib = load_library()
    ns = ctypes.c_int(0)
    ws = ctypes.c_size_t(0)
    _check(lib.rel_attn_decode_plan(B, L, Hq, Hkv, D, int(num_splits), int(window), int(rel_extent),
                                    ctypes.byref(ns), ctypes.byref(ws)))
    return ns.value, ws.value


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, r: Optional[torch.Tensor],
           P_cols: Optional[torch.Tensor], alpha: float, rel_extent: int, window: int = 0,
           log_scale: bool = False, num_splits: int = 0, return_lse: bool = True,
           workspace: Optional[torch.Tensor] = None
           ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Split-KV decode of one query token per sequence at position L-1.

    q [B,Hq,D], k/v cache [B,L,Hkv,D], r [B,Hq,d_r], P_cols [E,d_r].
    Returns out [B,Hq,D] and lse [B,Hq] fp32 (or None).
    """
    lib = load_library()
    dev = q.device
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    _need(q, "q", dt, dev, 3)
    _need(k, "k", dt, dev, 4)
    _need(v, "v", dt, dev, 4)
    B, Hq, D = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, L, Hkv, D) or v.shape != k.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    d_r = 0
    if rel_extent > 0:
        _need(r, "r", dt, dev, 3)
        _need(P_cols, "P_cols", dt, dev, 2)
        d_r = r.shape[2]
        if r.shape[:2] != (B, Hq):
            raise ValueError(f"r shape {tuple(r.shape)} does not match q")
        if P_cols.shape != (rel_extent, d_r):
            raise ValueError(f"P_cols must be [rel_extent={rel_extent}, d_r={d_r}], got {tuple(P_cols.shape)}")
    else:
        r = None
        P_cols = None
    ns, ws_bytes = decode_plan(B, L, Hq, Hkv, D, num_splits, window, rel_extent)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev) if return_lse else None
    _check(lib.rel_attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(r), _ptr(P_cols), _ptr(out), _ptr(lse),
                               _DTYPE_CODE[dt], B, L, Hq, Hkv, D, d_r, float(alpha), int(rel_extent),
                               int(window), 1 if log_scale else 0, ns, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(dev)))
    return out, lse


def decode_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, r: Optional[torch.Tensor],
                   P_cols: Optional[torch.Tensor], alpha: float, rel_extent: int, window: int = 0,
                   log_scale: bool = False, num_splits: int = 0, return_lse: bool = True,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None
                   ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``decode`` through rel_attn_decode_noalloc: no workspace, the library's
    fixed per-device scratch instead (calls that overlap on one GPU race).
    ``out`` / ``lse`` may be passed preallocated; otherwise they are created
    here (the C call itself allocates nothing); lse is skipped when
    ``return_lse`` is false and none is passed."""
    lib = load_library()
    dev = q.device
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    _need(q, "q", dt, dev, 3)
    _need(k, "k", dt, dev, 4)
    _need(v, "v", dt, dev, 4)
    B, Hq, D = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, L, Hkv, D) or v.shape != k.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    d_r = 0
    if rel_extent > 0:
        _need(r, "r", dt, dev, 3)
        _need(P_cols, "P_cols", dt, dev, 2)
        d_r = r.shape[2]
        if r.shape[:2] != (B, Hq):
            raise ValueError(f"r shape {tuple(r.shape)} does not match q")
        if P_cols.shape != (rel_extent, d_r):
            raise ValueError(f"P_cols must be [rel_extent={rel_extent}, d_r={d_r}], got {tuple(P_cols.shape)}")
    else:
        r = None
        P_cols = None
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", dt, dev, 3)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, 2)
    elif return_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    _check(lib.rel_attn_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(r), _ptr(P_cols), _ptr(out), _ptr(lse),
                                       _DTYPE_CODE[dt], B, L, Hq, Hkv, D, d_r, float(alpha), int(rel_extent),
                                       int(window), 1 if log_scale else 0, int(num_splits), _stream(dev)))
    return out, lse


def rel_logits(r: torch.Tensor, P_cols: torch.Tensor, log_scale: bool = False,
               seq_len: int = 0) -> torch.Tensor:
    """Dense relative logits s * r . P[:, d] for every d < E: r [n,H,d_r] -> [n,H,E] fp32."""
    lib = load_library()
    dev = r.device
    dt = r.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    _need(r, "r", dt, dev, 3)
    _need(P_cols, "P_cols", dt, dev, 2)
    n, H, d_r = r.shape
    E = P_cols.shape[0]
    if P_cols.shape[1] != d_r:
        raise ValueError("P_cols must be [E, d_r]")
    out = torch.empty(n, H, E, dtype=torch.float32, device=dev)
    _check(lib.rel_logits(_ptr(r), _ptr(P_cols), _ptr(out), _DTYPE_CODE[dt], n, H, d_r, E,
                          1 if log_scale else 0, int(seq_len if seq_len else n), _stream(dev)))
    return out


def decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, r: Optional[torch.Tensor],
                 P_cols: Optional[torch.Tensor], alpha: float, rel_extent: int, window: int, log_scale: bool,
                 kv_len: torch.Tensor, block_table: torch.Tensor, max_len: int, num_splits: int = 0,
                 return_lse: bool = True, workspace: Optional[torch.Tensor] = None
                 ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Split-KV decode over paged caches with per-sequence lengths (rel_attn_decode_paged).

    q [B,Hq,D], k_pages/v_pages [num_pages,page_size,Hkv,D], block_table
    [B,max_pages] and kv_len [B] (int32, device; each in [1, max_len]),
    r [B,Hq,d_r], P_cols [E,d_r].  Returns out [B,Hq,D] and lse [B,Hq] fp32.
    """
    lib = load_library()
    dev = q.device
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    _need(q, "q", dt, dev, 3)
    _need(k_pages, "k_pages", dt, dev, 4)
    _need(v_pages, "v_pages", dt, dev, 4)
    _need(kv_len, "kv_len", torch.int32, dev, 1)
    _need(block_table, "block_table", torch.int32, dev, 2)
    B, Hq, D = q.shape
    num_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if v_pages.shape != k_pages.shape:
        raise ValueError("v_pages shape differs from k_pages")
    if kv_len.shape[0] != B or block_table.shape[0] != B:
        raise ValueError("kv_len and block_table need one entry / row per sequence")
    d_r = 0
    if rel_extent > 0:
        _need(r, "r", dt, dev, 3)
        _need(P_cols, "P_cols", dt, dev, 2)
        d_r = r.shape[2]
    else:
        r = None
        P_cols = None
    ns, ws_bytes = decode_plan(B, max_len, Hq, Hkv, D, num_splits, window, rel_extent)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev) if return_lse else None
    _check(lib.rel_attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(r), _ptr(P_cols), _ptr(out),
                                     _ptr(lse), _DTYPE_CODE[dt], B, int(max_len), _ptr(kv_len), _ptr(block_table),
                                     block_table.shape[1], num_pages, page_size, Hq, Hkv, D, d_r, float(alpha),
                                     int(rel_extent), int(window), 1 if log_scale else 0, ns, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(dev)))
    return out, lse


def prologue(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, conv_k: torch.Tensor, conv_v: torch.Tensor,
             q_norm_w: torch.Tensor, k_norm_w: torch.Tensor, eps: float, q_start: torch.Tensor,
             kv_len: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
             block_table: Optional[torch.Tensor] = None, state_in: Optional[torch.Tensor] = None,
             state_out: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Attention prologue (rel_attn_prologue): K/V ShortConv, Q/K RMSNorm and the cache write.

    q [total_q,Hq,D], k/v [total_q,Hkv,D] raw projections packed by ``q_start``
    [B+1]; ``kv_len`` [B] (int32, device) sets each sequence's positions as in
    ``extend``.  conv_k/conv_v [Hkv*D, W]; q_norm_w/k_norm_w [D].  k_cache and
    v_cache are written in place (contiguous [B,cache_len,Hkv,D], or pages
    [num_pages,page_size,Hkv,D] with ``block_table`` [B,max_pages]).
    state_in/state_out [B,2,3,Hkv*D] carry the raw rows before / after the
    chunk.  Returns q_out [total_q,Hq,D] (``q`` itself may be passed as
    ``q_out``).
    """
    lib = load_library()
    dev = q.device
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    _need(q, "q", dt, dev, 3)
    _need(k, "k", dt, dev, 3)
    _need(v, "v", dt, dev, 3)
    _need(conv_k, "conv_k", dt, dev, 2)
    _need(conv_v, "conv_v", dt, dev, 2)
    _need(q_norm_w, "q_norm_w", dt, dev, 1)
    _need(k_norm_w, "k_norm_w", dt, dev, 1)
    _need(q_start, "q_start", torch.int32, dev, 1)
    _need(kv_len, "kv_len", torch.int32, dev, 1)
    _need(k_cache, "k_cache", dt, dev, 4)
    _need(v_cache, "v_cache", dt, dev, 4)
    total_q, Hq, D = q.shape
    Hkv = k.shape[1]
    B = kv_len.shape[0]
    if q_start.shape[0] != B + 1:
        raise ValueError(f"q_start must have B+1 = {B + 1} entries, got {q_start.shape[0]}")
    if k.shape != (total_q, Hkv, D) or v.shape != k.shape:
        raise ValueError(f"k and v must be [total_q={total_q}, Hkv, D={D}], got {tuple(k.shape)} and {tuple(v.shape)}")
    W = conv_k.shape[1]
    if conv_k.shape != (Hkv * D, W) or conv_v.shape != conv_k.shape:
        raise ValueError(f"conv_k and conv_v must be [Hkv*D={Hkv * D}, W], got {tuple(conv_k.shape)}")
    if q_norm_w.shape != (D,) or k_norm_w.shape != (D,):
        raise ValueError(f"q_norm_w and k_norm_w must be [D={D}]")
    if v_cache.shape != k_cache.shape:
        raise ValueError("v_cache shape differs from k_cache")
    if block_table is None:
        cache_len, max_pages, num_pages, page_size = k_cache.shape[1], 0, 0, 0
        if k_cache.shape[0] != B:
            raise ValueError(f"contiguous caches must be [B={B}, cache_len, Hkv, D], got {tuple(k_cache.shape)}")
    else:
        _need(block_table, "block_table", torch.int32, dev, 2)
        if block_table.shape[0] != B:
            raise ValueError(f"block_table must be [B={B}, max_pages], got {tuple(block_table.shape)}")
        cache_len, max_pages, num_pages, page_size = 0, block_table.shape[1], k_cache.shape[0], k_cache.shape[1]
    for name, st in (("state_in", state_in), ("state_out", state_out)):
        if st is not None:
            _need(st, name, dt, dev, 4)
            if st.shape != (B, 2, 3, Hkv * D):
                raise ValueError(f"{name} must be [B={B}, 2, 3, Hkv*D={Hkv * D}], got {tuple(st.shape)}")
    if q_out is None:
        q_out = torch.empty_like(q)
    else:
        _need(q_out, "q_out", dt, dev, 3)
    _check(lib.rel_attn_prologue(_ptr(q), _ptr(k), _ptr(v), _ptr(conv_k), _ptr(conv_v), _ptr(q_norm_w),
                                 _ptr(k_norm_w), float(eps), _ptr(state_in), _ptr(state_out), _ptr(q_out),
                                 _ptr(k_cache), _ptr(v_cache), _DTYPE_CODE[dt], B, total_q, _ptr(q_start),
                                 _ptr(kv_len), cache_len, _ptr(block_table), max_pages, num_pages, page_size,
                                 Hq, Hkv, D, W, _stream(dev)))
    return q_out


def mx_quantize(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """MXFP8 of rows of 128 values (rel_mx_quantize): returns (codes uint8
    [..., 128], scales uint8 [..., 4])."""
    lib = load_library()
    dt = x.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    if not x.is_contiguous() or x.shape[-1] != 128:
        raise ValueError("x must be contiguous with a last dimension of 128")
    n = x.numel() // 128
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (4,), dtype=torch.uint8, device=x.device)
    _check(lib.rel_mx_quantize(_ptr(x), _ptr(codes), _ptr(scales), _DTYPE_CODE[dt], n, 128, _stream(x.device)))
    return codes, scales


def decode_mx(q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, v_codes: torch.Tensor,
              v_scales: torch.Tensor, r: Optional[torch.Tensor], P_cols: Optional[torch.Tensor], alpha: float,
              rel_extent: int, window: int = 0, log_scale: bool = False, L: Optional[int] = None,
              kv_len: Optional[torch.Tensor] = None, block_table: Optional[torch.Tensor] = None,
              num_splits: int = 0, return_lse: bool = True, workspace: Optional[torch.Tensor] = None
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Split-KV decode over MXFP8 caches (rel_attn_decode_mx).

    q [B,Hq,D] bf16.  Contiguous: codes [B,L,Hkv,D], scales [B,L,Hkv,D/32]
    (uint8).  Paged: codes [num_pages,page_size,Hkv,D], scales
    [num_pages,page_size,Hkv,D/32], ``block_table`` [B,max_pages] and
    ``kv_len`` [B] (int32, device), ``L`` the bound on kv_len.  Returns out
    [B,Hq,D] bf16 and lse [B,Hq] fp32.
    """
    lib = load_library()
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    for name, t in (("k_codes", k_codes), ("v_codes", v_codes), ("k_scales", k_scales), ("v_scales", v_scales)):
        _need(t, name, torch.uint8, dev, 4)
    B, Hq, D = q.shape
    Hkv = k_codes.shape[2]
    paged = block_table is not None
    if paged:
        _need(block_table, "block_table", torch.int32, dev, 2)
        _need(kv_len, "kv_len", torch.int32, dev, 1)
        if L is None:
            raise ValueError("paged caches need L, the bound on kv_len")
        max_pages, num_pages, page_size = block_table.shape[1], k_codes.shape[0], k_codes.shape[1]
    else:
        if kv_len is not None:
            raise ValueError("kv_len is for paged caches")
        L = k_codes.shape[1]
        max_pages = num_pages = page_size = 0
    if v_codes.shape != k_codes.shape or k_scales.shape != k_codes.shape[:3] + (D // 32,) or \
            v_scales.shape != k_scales.shape:
        raise ValueError("code and scale shapes do not match")
    d_r = 0
    if rel_extent > 0:
        _need(r, "r", torch.bfloat16, dev, 3)
        _need(P_cols, "P_cols", torch.bfloat16, dev, 2)
        d_r = r.shape[2]
    else:
        r = None
        P_cols = None
    ns, ws_bytes = decode_plan(B, L, Hq, Hkv, D, num_splits, window, rel_extent)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev) if return_lse else None
    _check(lib.rel_attn_decode_mx(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales), _ptr(r),
                                  _ptr(P_cols), _ptr(out), _ptr(lse), B, int(L), _ptr(kv_len), _ptr(block_table),
                                  max_pages, num_pages, page_size, Hq, Hkv, D, d_r, float(alpha), int(rel_extent),
                                  int(window), 1 if log_scale else 0, ns, _ptr(workspace), workspace.numel(),
                                  _stream(dev)))
    return out, lse


def prologue_mx(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, conv_k: torch.Tensor, conv_v: torch.Tensor,
                q_norm_w: torch.Tensor, k_norm_w: torch.Tensor, eps: float, q_start: torch.Tensor,
                kv_len: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, v_codes: torch.Tensor,
                v_scales: torch.Tensor, block_table: Optional[torch.Tensor] = None,
                state_in: Optional[torch.Tensor] = None, state_out: Optional[torch.Tensor] = None,
                q_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The attention prologue writing MXFP8 caches (rel_attn_prologue_mx); bf16
    inputs; codes [..,Hkv,128] and scales [..,Hkv,4] uint8, written in place."""
    lib = load_library()
    dev = q.device
    dt = torch.bfloat16
    for name, t, nd in (("q", q, 3), ("k", k, 3), ("v", v, 3), ("conv_k", conv_k, 2), ("conv_v", conv_v, 2),
                        ("q_norm_w", q_norm_w, 1), ("k_norm_w", k_norm_w, 1)):
        _need(t, name, dt, dev, nd)
    for name, t in (("k_codes", k_codes), ("v_codes", v_codes), ("k_scales", k_scales), ("v_scales", v_scales)):
        _need(t, name, torch.uint8, dev, 4)
    _need(q_start, "q_start", torch.int32, dev, 1)
    _need(kv_len, "kv_len", torch.int32, dev, 1)
    total_q, Hq, D = q.shape
    Hkv = k.shape[1]
    B = kv_len.shape[0]
    W = conv_k.shape[1]
    if block_table is None:
        cache_len, max_pages, num_pages, page_size = k_codes.shape[1], 0, 0, 0
    else:
        _need(block_table, "block_table", torch.int32, dev, 2)
        cache_len, max_pages, num_pages, page_size = 0, block_table.shape[1], k_codes.shape[0], k_codes.shape[1]
    for name, st in (("state_in", state_in), ("state_out", state_out)):
        if st is not None:
            _need(st, name, dt, dev, 4)
    if q_out is None:
        q_out = torch.empty_like(q)
    _check(lib.rel_attn_prologue_mx(_ptr(q), _ptr(k), _ptr(v), _ptr(conv_k), _ptr(conv_v), _ptr(q_norm_w),
                                    _ptr(k_norm_w), float(eps), _ptr(state_in), _ptr(state_out), _ptr(q_out),
                                    _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales), B, total_q,
                                    _ptr(q_start), _ptr(kv_len), cache_len, _ptr(block_table), max_pages, num_pages,
                                    page_size, Hq, Hkv, D, W, _stream(dev)))
    return q_out


def backward_plan(B: int, T: int, Hq: int, Hkv: int, D: int = 128, head_splits: int = 0) -> Tuple[int, int]:
    """(head_splits, workspace bytes) of a backward call of this shape."""
    lib = load_library()
    ns = ctypes.c_int(0)
    wb = ctypes.c_size_t(0)
    _check(lib.rel_attn_backward_plan(B, T, Hq, Hkv, D, head_splits, ctypes.byref(ns), ctypes.byref(wb)))
    return ns.value, wb.value


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, r: Optional[torch.Tensor],
             P_cols: Optional[torch.Tensor], out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
             alpha: float, rel_extent: int, window: int = 0, log_scale: bool = False, head_splits: int = 0,
             workspace: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv, dr) of sum(dout * out) for a bf16 prefill call.

    q, out, dout [B,T,Hq,D]; k, v [B,T,Hkv,D]; r [B,T,Hq,d_r]; P_cols [E,d_r];
    lse [B,Hq,T] fp32 from the forward.  dr is None when rel_extent == 0.
    """
    lib = load_library()
    dev = q.device
    dt = q.dtype
    if dt != torch.bfloat16:
        raise TypeError(f"backward supports bfloat16 only, got {dt}")
    _need(q, "q", dt, dev, 4)
    _need(k, "k", dt, dev, 4)
    _need(v, "v", dt, dev, 4)
    _need(out, "out", dt, dev, 4)
    _need(dout, "dout", dt, dev, 4)
    _need(lse, "lse", torch.float32, dev, 3)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, T, Hkv, D) or v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q/k/v/out/dout shapes do not agree")
    if lse.shape != (B, Hq, T):
        raise ValueError(f"lse must be [B, Hq, T] = {(B, Hq, T)}, got {tuple(lse.shape)}")
    d_r = 0
    if rel_extent > 0:
        _need(r, "r", dt, dev, 4)
        _need(P_cols, "P_cols", dt, dev, 2)
        d_r = r.shape[3]
        if r.shape[:3] != (B, T, Hq):
            raise ValueError(f"r shape {tuple(r.shape)} does not match q")
        if P_cols.shape != (rel_extent, d_r):
            raise ValueError(f"P_cols must be [rel_extent={rel_extent}, d_r={d_r}], got {tuple(P_cols.shape)}")
    else:
        r = None
        P_cols = None
    ns, ws_bytes = backward_plan(B, T, Hq, Hkv, D, head_splits)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dr = torch.empty(B, T, Hq, d_r, dtype=dt, device=dev) if rel_extent > 0 else None
    _check(lib.rel_attn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(r), _ptr(P_cols), _ptr(out), _ptr(dout), _ptr(lse),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dr), _DTYPE_CODE[dt], B, T, Hq, Hkv, D, d_r,
                                 float(alpha), int(rel_extent), int(window), 1 if log_scale else 0, ns,
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)))
    return dq, dk, dv, dr
