"""Thin ctypes binding of libattn (include/attn.h): argument marshalling only.

torch supplies device memory and the current stream; every computation runs in the HIP
kernels behind the C ABI.  There is no fallback: if the library is missing or a call
returns an error status, a RuntimeError is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_OK = 0


class AttnTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_s", ctypes.c_int64),
                ("stride_h", ctypes.c_int64)]


# element type codes of include/attn.h
DTYPE_BF16, DTYPE_F32, DTYPE_F16 = 0, 1, 2
_DT16 = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16}


class AttnShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("total", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class AttnChunkShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Sq", ctypes.c_int32), ("Sk", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class AttnKernelTime(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char_p), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


class AttnDecodeShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class AttnPagedShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("max_q", ctypes.c_int32), ("total_q", ctypes.c_int32),
                ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32)]


_lib = None

EXPORTS = ("attn_fwd", "attn_bwd", "attn_fwd_chunk", "attn_bwd_chunk", "attn_lse_merge", "attn_fwd_chunk_merge",
           "paged_decode", "paged_kv_append", "paged_kv_gather", "attn_debug",
           "attn_fwd_workspace_bytes", "attn_bwd_workspace_bytes", "attn_bwd_chunk_workspace_bytes",
           "paged_decode_workspace_bytes", "attn_status_str", "attn_last_hip_error", "attn_version",
           "attn_profile", "attn_profile_read", "attn_count_restarts", "paged_decode_noalloc",
           "paged_decode_noalloc_max_bytes", "attn_peak_probe", "attn_fwd_paged", "attn_fwd_paged_split", "attn_fwd_paged_workspace_bytes",
           "paged_decode_contiguous",
           "paged_decode_graphs_create", "paged_decode_graphs_launch", "paged_decode_graphs_destroy")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so (built by ``scaled_dot_product_tiled_amd.build``) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libattn.so not found at {path}; build it with "
                           "`python -m scaled_dot_product_tiled_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.attn_fwd.argtypes = [P(AttnShape), AttnTensor, AttnTensor, AttnTensor, ctypes.c_float, ctypes.c_int,
                             ctypes.c_int, ctypes.c_float, vp, vp, AttnTensor, vp, vp, sz, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [P(AttnShape), AttnTensor, AttnTensor, AttnTensor, AttnTensor, vp, AttnTensor,
                             ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp, AttnTensor,
                             AttnTensor, AttnTensor, vp, sz, vp]
    lib.attn_bwd.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.attn_fwd_chunk.argtypes = [P(AttnChunkShape), AttnTensor, AttnTensor, AttnTensor, ctypes.c_float, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_float, i64, i64, AttnTensor, ctypes.c_int, vp, vp]
    lib.attn_fwd_chunk.restype = ctypes.c_int
    lib.attn_bwd_chunk.argtypes = [P(AttnChunkShape), AttnTensor, AttnTensor, AttnTensor, AttnTensor, vp, AttnTensor,
                                   ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_float, i64, i64, AttnTensor,
                                   AttnTensor, AttnTensor, ctypes.c_int, vp, sz, vp]
    lib.attn_bwd_chunk.restype = ctypes.c_int
    lib.attn_bwd_chunk_workspace_bytes.argtypes = [P(AttnChunkShape), ctypes.c_int, ctypes.c_int, i64, i64]
    lib.attn_bwd_chunk_workspace_bytes.restype = sz
    lib.attn_lse_merge.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, AttnTensor, vp,
                                   AttnTensor, vp, AttnTensor, ctypes.c_int, vp]
    lib.attn_lse_merge.restype = ctypes.c_int
    lib.attn_fwd_chunk_merge.argtypes = [P(AttnChunkShape), AttnTensor, AttnTensor, AttnTensor, ctypes.c_float,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_float, i64, i64, AttnTensor, vp,
                                         AttnTensor, vp]
    lib.attn_fwd_chunk_merge.restype = ctypes.c_int
    lib.paged_decode.argtypes = [P(AttnDecodeShape), vp, ctypes.c_int64, ctypes.c_int64, AttnTensor, AttnTensor,
                                 vp, vp, ctypes.c_float, ctypes.c_float, vp, ctypes.c_int64, ctypes.c_int64, vp, sz,
                                 vp]
    lib.paged_decode.restype = ctypes.c_int
    lib.paged_decode_noalloc.argtypes = [P(AttnDecodeShape), vp, ctypes.c_int64, ctypes.c_int64, AttnTensor,
                                         AttnTensor, vp, vp, ctypes.c_float, ctypes.c_float, vp, ctypes.c_int64,
                                         ctypes.c_int64, vp]
    lib.paged_decode_noalloc.restype = ctypes.c_int
    lib.paged_decode_contiguous.argtypes = lib.paged_decode.argtypes
    lib.paged_decode_contiguous.restype = ctypes.c_int
    lib.paged_decode_graphs_create.argtypes = [P(AttnDecodeShape), vp, ctypes.c_int32, vp, ctypes.c_int64,
                                               ctypes.c_int64, AttnTensor, AttnTensor, AttnTensor, AttnTensor, vp, vp,
                                               ctypes.c_float, ctypes.c_float, vp, ctypes.c_int64, ctypes.c_int64, vp,
                                               sz, vp, P(vp)]
    lib.paged_decode_graphs_create.restype = ctypes.c_int
    lib.paged_decode_graphs_launch.argtypes = [vp, ctypes.c_int32, vp, P(ctypes.c_int32)]
    lib.paged_decode_graphs_launch.restype = ctypes.c_int
    lib.paged_decode_graphs_destroy.argtypes = [vp]
    lib.paged_decode_graphs_destroy.restype = None
    lib.paged_decode_noalloc_max_bytes.argtypes = []
    lib.paged_decode_noalloc_max_bytes.restype = sz
    lib.paged_kv_append.argtypes = [P(AttnDecodeShape), ctypes.c_int32, AttnTensor, AttnTensor, AttnTensor, AttnTensor,
                                    vp, vp, vp]
    lib.paged_kv_append.restype = ctypes.c_int
    lib.paged_kv_gather.argtypes = [P(AttnDecodeShape), ctypes.c_int32, AttnTensor, AttnTensor, vp, vp, AttnTensor,
                                    AttnTensor, vp]
    lib.paged_kv_gather.restype = ctypes.c_int
    lib.attn_fwd_paged.argtypes = [P(AttnPagedShape), AttnTensor, AttnTensor, AttnTensor, vp, vp, vp, ctypes.c_float,
                                   ctypes.c_int, ctypes.c_float, AttnTensor, vp, vp]
    lib.attn_fwd_paged.restype = ctypes.c_int
    lib.attn_fwd_paged_workspace_bytes.argtypes = [P(AttnPagedShape)]
    lib.attn_fwd_paged_workspace_bytes.restype = sz
    lib.attn_fwd_paged_split.argtypes = [P(AttnPagedShape), AttnTensor, AttnTensor, AttnTensor, vp, vp, vp,
                                         ctypes.c_float, ctypes.c_int, ctypes.c_float, AttnTensor, vp, vp, sz, vp]
    lib.attn_fwd_paged_split.restype = ctypes.c_int
    lib.attn_debug.argtypes = [ctypes.c_int]
    lib.attn_debug.restype = ctypes.c_int
    lib.attn_fwd_workspace_bytes.argtypes = [P(AttnShape), ctypes.c_int]
    lib.attn_fwd_workspace_bytes.restype = sz
    lib.attn_bwd_workspace_bytes.argtypes = [P(AttnShape), ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.paged_decode_workspace_bytes.argtypes = [P(AttnDecodeShape)]
    lib.paged_decode_workspace_bytes.restype = sz
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = ctypes.c_int
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    lib.attn_peak_probe.argtypes = [ctypes.c_int, vp, sz, ctypes.c_int, vp]
    lib.attn_peak_probe.restype = ctypes.c_int
    lib.attn_count_restarts.argtypes = [vp]
    lib.attn_count_restarts.restype = ctypes.c_int
    lib.attn_profile.argtypes = [ctypes.c_int]
    lib.attn_profile.restype = ctypes.c_int
    lib.attn_profile_read.argtypes = [P(AttnKernelTime), ctypes.c_int]
    lib.attn_profile_read.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int, what: str) -> None:
    if status != ATTN_OK:
        lib = load_library()
        msg = lib.attn_status_str(status).decode()
        hip = lib.attn_last_hip_error()
        raise RuntimeError(f"{what} failed: status {status} ({msg})" + (f", hip error {hip}" if status == 4 else ""))


def _half(t: torch.Tensor, name: str, like: Optional[torch.dtype] = None) -> None:
    """A 16-bit (bfloat16 or float16) device tensor with a contiguous last dimension, of the
    same type as the call's other tensors (like)."""
    if not isinstance(t, torch.Tensor) or t.dtype not in _DT16 or not t.is_cuda:
        raise TypeError(f"{name} must be a bfloat16 or float16 CUDA/HIP tensor")
    if like is not None and t.dtype != like:
        raise TypeError(f"{name} is {t.dtype}, the call's tensors are {like}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: the head_dim dimension must be contiguous")


def _expect(t: torch.Tensor, shape, name: str) -> None:
    """Every tensor's sizes are checked against the call's shape; the library reads each tensor
    through its own strides, so a mismatched tensor would be read past its end."""
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != torch.device("cuda", torch.cuda.current_device()):
        raise ValueError(f"{name} must live on the current device")


def _check_attn_shapes(shape, packed, q, k, v, lse=None, o=None, **grads) -> None:
    """q, o, dout, dq: (B,S,Hq,D) or packed (T,Hq,D); k, v, dk, dv: (B,S,Hkv,D) or (T,Hkv,D)."""
    if packed:
        qs, ks = (shape.total, shape.Hq, shape.D), (shape.total, shape.Hkv, shape.D)
        ls = (shape.Hq, shape.total)
    else:
        qs, ks = (shape.B, shape.S, shape.Hq, shape.D), (shape.B, shape.S, shape.Hkv, shape.D)
        ls = (shape.B, shape.Hq, shape.S)
    _expect(k, ks, "k")
    _expect(v, ks, "v")
    for n, t in (("o", o), ("dout", grads.get("dout")), ("dq", grads.get("dq"))):
        if t is not None:
            _expect(t, qs, n)
            _half(t, n, q.dtype)
    for n, t in (("dk", grads.get("dk")), ("dv", grads.get("dv"))):
        if t is not None:
            _expect(t, ks, n)
            _half(t, n, q.dtype)
    if lse is not None:
        _expect(lse, ls, "lse")
        if lse.dtype != torch.float32 or not lse.is_contiguous():
            raise TypeError("lse must be a contiguous float32 tensor")


def _tensor(t: torch.Tensor, packed: bool) -> AttnTensor:
    if packed:   # (T, H, D)
        return AttnTensor(t.data_ptr(), 0, t.stride(0), t.stride(1))
    return AttnTensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _shape(q, k, cu_seqlens, pad_mask, max_seqlen):
    packed = cu_seqlens is not None
    if packed:
        T, Hq, D = q.shape
        B = cu_seqlens.numel() - 1
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with cu_seqlens")
        S = int(max_seqlen)
    else:
        B, S, Hq, D = q.shape
        T = 0
    Hkv = k.shape[-2]
    if pad_mask is not None and tuple(pad_mask.shape) != (B, S):
        raise ValueError(f"pad_mask must be (B, S) = {(B, S)}, got {tuple(pad_mask.shape)}")
    return AttnShape(B, S, T, Hq, Hkv, D, _DT16[q.dtype]), packed, (2 if packed else (1 if pad_mask is not None else 0))


def _meta_ptrs(cu_seqlens, pad_mask):
    cu = None
    pm = None
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or not cu_seqlens.is_contiguous():
            raise TypeError("cu_seqlens must be a contiguous int32 device tensor")
        cu = cu_seqlens.data_ptr()
    if pad_mask is not None:
        if pad_mask.dtype not in (torch.bool, torch.uint8) or not pad_mask.is_cuda or not pad_mask.is_contiguous():
            raise TypeError("pad_mask must be a contiguous bool/uint8 device tensor")
        pm = pad_mask.data_ptr()
    return cu, pm


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None, causal: bool = True,
             window: int = 0, cu_seqlens: Optional[torch.Tensor] = None, pad_mask: Optional[torch.Tensor] = None,
             max_seqlen: Optional[int] = None, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None, softcap: float = 0.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """O, LSE of causal grouped-query attention.  q (B,S,Hq,D), k/v (B,S,Hkv,D); with cu_seqlens the
    rows are packed: q (T,Hq,D), k/v (T,Hkv,D), LSE (Hq,T).  Returns (O, LSE fp32)."""
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _half(t, n, q.dtype)
    shape, packed, varlen = _shape(q, k, cu_seqlens, pad_mask, max_seqlen)
    if scale is None:
        scale = 1.0 / math.sqrt(shape.D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse_shape = (shape.Hq, shape.total) if packed else (shape.B, shape.Hq, shape.S)
        lse = torch.empty(lse_shape, device=q.device, dtype=torch.float32)
    _check_attn_shapes(shape, packed, q, k, v, lse=lse, o=out)
    cu, pm = _meta_ptrs(cu_seqlens, pad_mask)
    nbytes = lib.attn_fwd_workspace_bytes(ctypes.byref(shape), varlen)
    ws = torch.empty(max(nbytes, 1), device=q.device, dtype=torch.uint8)
    st = lib.attn_fwd(ctypes.byref(shape), _tensor(q, packed), _tensor(k, packed), _tensor(v, packed), float(scale),
                      int(bool(causal)), int(window), float(softcap), cu, pm, _tensor(out, packed), lse.data_ptr(),
                      ws.data_ptr() if nbytes else None, nbytes, _stream())
    _check(st, "attn_fwd")
    return out, lse


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, scale: Optional[float] = None, causal: bool = True, window: int = 0,
             cu_seqlens: Optional[torch.Tensor] = None, pad_mask: Optional[torch.Tensor] = None,
             max_seqlen: Optional[int] = None, dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None, softcap: float = 0.0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dQ, dK, dV of sum(O * dO), from attn_fwd's O and LSE."""
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _half(t, n, q.dtype)
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    shape, packed, varlen = _shape(q, k, cu_seqlens, pad_mask, max_seqlen)
    if scale is None:
        scale = 1.0 / math.sqrt(shape.D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_attn_shapes(shape, packed, q, k, v, lse=lse, o=o, dout=dout, dq=dq, dk=dk, dv=dv)
    cu, pm = _meta_ptrs(cu_seqlens, pad_mask)
    nbytes = lib.attn_bwd_workspace_bytes(ctypes.byref(shape), varlen, int(bool(causal)), int(window))
    ws = torch.empty(max(nbytes, 1), device=q.device, dtype=torch.uint8)
    st = lib.attn_bwd(ctypes.byref(shape), _tensor(q, packed), _tensor(k, packed), _tensor(v, packed),
                      _tensor(o, packed), lse.data_ptr(), _tensor(dout, packed), float(scale), int(bool(causal)),
                      int(window), float(softcap), cu, pm, _tensor(dq, packed), _tensor(dk, packed), _tensor(dv, packed),
                      ws.data_ptr() if nbytes else None, nbytes, _stream())
    _check(st, "attn_bwd")
    return dq, dk, dv


def _chunk_shape(q, k):
    B, Sq, Hq, D = q.shape
    return AttnChunkShape(B, Sq, k.shape[1], Hq, k.shape[2], D, _DT16[q.dtype])


def _check_chunk_shapes(shape, q, k, v, lse=None, o=None, **grads) -> None:
    """q, o, dout, dq: (B,Sq,Hq,D); k, v, dk, dv: (B,Sk,Hkv,D); lse (B,Hq,Sq)."""
    qs = (shape.B, shape.Sq, shape.Hq, shape.D)
    ks = (shape.B, shape.Sk, shape.Hkv, shape.D)
    _expect(q, qs, "q")
    for n, t in (("k", k), ("v", v), ("dk", grads.get("dk")), ("dv", grads.get("dv"))):
        if t is not None:
            _expect(t, ks, n)
    for n, t in (("o", o), ("dout", grads.get("dout")), ("dq", grads.get("dq"))):
        if t is not None:
            _expect(t, qs, n)
    if lse is not None:
        _expect(lse, (shape.B, shape.Hq, shape.Sq), "lse")
        if lse.dtype != torch.float32 or not lse.is_contiguous():
            raise TypeError("lse must be a contiguous float32 tensor")


def attn_fwd_chunk(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_pos0: int, k_pos0: int,
                   scale: Optional[float] = None, causal: bool = True, window: int = 0,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   out_dtype: torch.dtype = torch.float32, softcap: float = 0.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Partial O, LSE of a query chunk q (B,Sq,Hq,D) at positions q_pos0.. against one key/value chunk
    k/v (B,Sk,Hkv,D) at positions k_pos0..; rows that see no key get O = 0, LSE = -inf.  O is fp32
    (a partial for attn_lse_merge) unless out_dtype is the inputs' 16-bit type."""
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _half(t, n, q.dtype)
    shape = _chunk_shape(q, k)
    if scale is None:
        scale = 1.0 / math.sqrt(shape.D)
    if out is None:
        out = torch.empty(tuple(q.shape), device=q.device, dtype=out_dtype)
    if out.dtype not in (torch.float32, q.dtype) or out.stride(-1) != 1 or not out.is_cuda:
        raise TypeError(f"out must be a float32 or {q.dtype} device tensor with a contiguous last dimension")
    if lse is None:
        lse = torch.empty((shape.B, shape.Hq, shape.Sq), device=q.device, dtype=torch.float32)
    _check_chunk_shapes(shape, q, k, v, lse=lse, o=out)
    st = lib.attn_fwd_chunk(ctypes.byref(shape), _tensor(q, False), _tensor(k, False), _tensor(v, False),
                            float(scale), int(bool(causal)), int(window), float(softcap), int(q_pos0), int(k_pos0),
                            _tensor(out, False), DTYPE_F32 if out.dtype == torch.float32 else _DT16[out.dtype],
                            lse.data_ptr(), _stream())
    _check(st, "attn_fwd_chunk")
    return out, lse


def attn_bwd_chunk_workspace_bytes(q: torch.Tensor, k: torch.Tensor, q_pos0: int, k_pos0: int, causal: bool = True,
                                   window: int = 0) -> int:
    """Workspace bytes attn_bwd_chunk needs for this chunk pair (q (B,Sq,Hq,D), k (B,Sk,Hkv,D))."""
    shape = _chunk_shape(q, k)
    return int(load_library().attn_bwd_chunk_workspace_bytes(ctypes.byref(shape), int(bool(causal)), int(window),
                                                             int(q_pos0), int(k_pos0)))


def attn_bwd_chunk(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                   dout: torch.Tensor, q_pos0: int, k_pos0: int, scale: Optional[float] = None,
                   causal: bool = True, window: int = 0, dq: Optional[torch.Tensor] = None,
                   dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
                   accumulate: bool = False, workspace: Optional[torch.Tensor] = None,
                   softcap: float = 0.0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradient parts dQ (B,Sq,Hq,D), dK, dV (B,Sk,Hkv,D) of one chunk pair, from the rows' final O and
    LSE (merged over all their key chunks) and dO.  accumulate=False writes the parts in the inputs'
    16-bit type (new tensors unless given); accumulate=True adds them to the given fp32 dq, dk, dv."""
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _half(t, n, q.dtype)
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    shape = _chunk_shape(q, k)
    if scale is None:
        scale = 1.0 / math.sqrt(shape.D)
    if accumulate:
        if dq is None or dk is None or dv is None:
            raise ValueError("accumulate=True needs the fp32 accumulators dq, dk, dv")
        for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            if t.dtype != torch.float32 or not t.is_cuda or t.stride(-1) != 1:
                raise TypeError(f"{n} must be a float32 device tensor with a contiguous last dimension")
    else:
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            _half(t, n, q.dtype)
    _check_chunk_shapes(shape, q, k, v, lse=lse, o=o, dout=dout, dq=dq, dk=dk, dv=dv)
    c, w = int(bool(causal)), int(window)
    nbytes = lib.attn_bwd_chunk_workspace_bytes(ctypes.byref(shape), c, w, int(q_pos0), int(k_pos0))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), device=q.device, dtype=torch.uint8)
    st = lib.attn_bwd_chunk(ctypes.byref(shape), _tensor(q, False), _tensor(k, False), _tensor(v, False),
                            _tensor(o, False), lse.data_ptr(), _tensor(dout, False), float(scale), c, w,
                            float(softcap), int(q_pos0), int(k_pos0), _tensor(dq, False), _tensor(dk, False), _tensor(dv, False),
                            DTYPE_F32 if accumulate else _DT16[q.dtype], workspace.data_ptr() if nbytes else None,
                            nbytes, _stream())
    _check(st, "attn_bwd_chunk")
    return dq, dk, dv


def attn_lse_merge(o: torch.Tensor, lse: torch.Tensor, o_part: torch.Tensor, lse_part: torch.Tensor,
                   out: Optional[torch.Tensor] = None) -> None:
    """In place: (o, lse) <- log-sum-exp merge of (o, lse) and (o_part, lse_part); o, o_part (B,S,H,D) fp32,
    lse, lse_part (B,H,S).  With out (B,S,H,D) bf16, the merged O rounded to bf16 is written there too."""
    lib = load_library()
    for t, n in ((o, "o"), (o_part, "o_part")):
        if t.dtype != torch.float32 or not t.is_cuda or t.stride(-1) != 1:
            raise TypeError(f"{n} must be a float32 device tensor with a contiguous last dimension")
    for t, n in ((lse, "lse"), (lse_part, "lse_part")):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise TypeError(f"{n} must be a contiguous float32 device tensor")
    B, S, H, D = o.shape
    _expect(o_part, (B, S, H, D), "o_part")
    _expect(lse, (B, H, S), "lse")
    _expect(lse_part, (B, H, S), "lse_part")
    if out is not None:
        _half(out, "out")
        _expect(out, (B, S, H, D), "out")
    st = lib.attn_lse_merge(B, S, H, D, _tensor(o, False), lse.data_ptr(), _tensor(o_part, False),
                            lse_part.data_ptr(), _tensor(out, False) if out is not None else AttnTensor(None, 0, 0, 0),
                            _DT16[out.dtype] if out is not None else DTYPE_BF16, _stream())
    _check(st, "attn_lse_merge")


def attn_fwd_chunk_merge(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_pos0: int, k_pos0: int,
                         o: torch.Tensor, lse: torch.Tensor, scale: Optional[float] = None, causal: bool = True,
                         window: int = 0, out: Optional[torch.Tensor] = None, softcap: float = 0.0) -> None:
    """In place: (o, lse) <- log-sum-exp merge of the running (o, lse) (fp32 (B,Sq,Hq,D), (B,Hq,Sq)) and
    the partial of the query chunk q at positions q_pos0.. against the key/value chunk k/v at
    k_pos0.. (attn_fwd_chunk then attn_lse_merge in one kernel).  Rows with lse = -inf take the
    partial whatever o holds.  With out (B,Sq,Hq,D) in q's dtype, the merged O is rounded into it."""
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _half(t, n, q.dtype)
    shape = _chunk_shape(q, k)
    if scale is None:
        scale = 1.0 / math.sqrt(shape.D)
    if o.dtype != torch.float32 or o.stride(-1) != 1 or not o.is_cuda:
        raise TypeError("o must be a float32 device tensor with a contiguous last dimension")
    if out is not None:
        _half(out, "out", q.dtype)
        _expect(out, tuple(q.shape), "out")
    _check_chunk_shapes(shape, q, k, v, lse=lse, o=o)
    st = lib.attn_fwd_chunk_merge(ctypes.byref(shape), _tensor(q, False), _tensor(k, False), _tensor(v, False),
                                  float(scale), int(bool(causal)), int(window), float(softcap), int(q_pos0),
                                  int(k_pos0), _tensor(o, False), lse.data_ptr(),
                                  _tensor(out, False) if out is not None else AttnTensor(None, 0, 0, 0), _stream())
    _check(st, "attn_fwd_chunk_merge")


def _decode_args(q, k_cache, v_cache, block_table, ctx_lens, scale, out):
    """Checks and marshals the arguments paged_decode and paged_decode_noalloc share."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _half(t, n, q.dtype)
    for t, n in ((block_table, "block_table"), (ctx_lens, "ctx_lens")):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous int32 device tensor")
    B, Hq, D = q.shape
    num_pages, page_size, Hkv, _ = k_cache.shape
    shape = AttnDecodeShape(B, Hq, Hkv, D, page_size, num_pages, block_table.shape[1], _DT16[q.dtype])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        raise ValueError("out is required")
    _half(out, "out", q.dtype)
    _expect(v_cache, tuple(k_cache.shape), "v_cache")
    _expect(out, (B, Hq, D), "out")
    _expect(ctx_lens, (B,), "ctx_lens")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be (B, max_pages_per_seq), got {tuple(block_table.shape)}")
    if k_cache.shape[3] != D:
        raise ValueError("k_cache head_dim differs from q's")
    return shape, float(scale)


def paged_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                         ctx_lens: torch.Tensor, out: torch.Tensor, scale: Optional[float] = None,
                         softcap: float = 0.0) -> torch.Tensor:
    """paged_decode without a workspace (the library's fixed device scratch holds the partials);
    out (B,Hq,D) is required, so that the call allocates nothing."""
    lib = load_library()
    shape, scale = _decode_args(q, k_cache, v_cache, block_table, ctx_lens, scale, out)
    st = lib.paged_decode_noalloc(ctypes.byref(shape), q.data_ptr(), q.stride(0), q.stride(1),
                                  AttnTensor(k_cache.data_ptr(), k_cache.stride(0), k_cache.stride(1),
                                             k_cache.stride(2)),
                                  AttnTensor(v_cache.data_ptr(), v_cache.stride(0), v_cache.stride(1),
                                             v_cache.stride(2)),
                                  block_table.data_ptr(), ctx_lens.data_ptr(), scale, float(softcap), out.data_ptr(),
                                  out.stride(0), out.stride(1), _stream())
    _check(st, "paged_decode_noalloc")
    return out


def paged_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                 ctx_lens: torch.Tensor, scale: Optional[float] = None,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 softcap: float = 0.0) -> torch.Tensor:
    """O (B,Hq,D) of one query token per sequence against a paged cache (num_pages, page_size, Hkv, D)."""
    return _decode_call("paged_decode", q, k_cache, v_cache, block_table, ctx_lens, scale, out, workspace, softcap)


def paged_decode_contiguous(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, first_page: torch.Tensor,
                            ctx_lens: torch.Tensor, max_pages_per_seq: int, scale: Optional[float] = None,
                            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                            softcap: float = 0.0) -> torch.Tensor:
    """paged_decode for caches whose sequences hold consecutive pages: logical page p of sequence b is
    physical page first_page[b] + p (first_page (B,) int32); contexts are bounded by max_pages_per_seq."""
    if first_page.dim() != 1:
        raise ValueError("first_page must be (B,)")
    return _decode_call("paged_decode_contiguous", q, k_cache, v_cache, first_page, ctx_lens, scale, out, workspace,
                        softcap, max_pages=int(max_pages_per_seq))


def _decode_call(fn, q, k_cache, v_cache, table, ctx_lens, scale, out, workspace, softcap, max_pages=None):
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    if max_pages is None:
        shape, scale = _decode_args(q, k_cache, v_cache, table, ctx_lens, scale, out)
    else:   # a (B,) first-page array in place of the table
        shape, scale = _decode_args(q, k_cache, v_cache, table.view(-1, 1), ctx_lens, scale, out)
        shape.max_pages_per_seq = max_pages
    nbytes = lib.paged_decode_workspace_bytes(ctypes.byref(shape))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), device=q.device, dtype=torch.uint8)
    st = getattr(lib, fn)(ctypes.byref(shape), q.data_ptr(), q.stride(0), q.stride(1),
                          AttnTensor(k_cache.data_ptr(), k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)),
                          AttnTensor(v_cache.data_ptr(), v_cache.stride(0), v_cache.stride(1), v_cache.stride(2)),
                          table.data_ptr(), ctx_lens.data_ptr(), scale, float(softcap), out.data_ptr(), out.stride(0),
                          out.stride(1), workspace.data_ptr(), nbytes, _stream())
    _check(st, fn)
    return out


class DecodeGraphs:
    """Captured decode steps, one HIP graph per batch bucket (paged_decode_graphs_create), over fixed
    buffers: q (Bmax,Hq,D), caches, block_table (Bmax, max_pages), ctx_lens (Bmax,), out (Bmax,Hq,D)
    and, when given, the current token's k_new / v_new (Bmax,1,Hkv,D) appended before each decode.
    launch(B) replays the smallest bucket >= B on the current stream and returns that bucket.  The
    tensors are kept referenced so the captured addresses stay valid."""

    def __init__(self, q, k_cache, v_cache, block_table, ctx_lens, out, buckets, scale=None, softcap=0.0,
                 k_new=None, v_new=None, stream=None):
        lib = load_library()
        shape, scale = _decode_args(q, k_cache, v_cache, block_table, ctx_lens, scale, out)
        if (k_new is None) != (v_new is None):
            raise ValueError("k_new and v_new go together")
        if k_new is not None:
            for t, n in ((k_new, "k_new"), (v_new, "v_new")):
                _half(t, n, q.dtype)
                _expect(t, (shape.B, 1, shape.Hkv, shape.D), n)
        nbytes = lib.paged_decode_workspace_bytes(ctypes.byref(shape))
        self.workspace = torch.empty(max(nbytes, 1), device=q.device, dtype=torch.uint8)
        self._keep = (q, k_cache, v_cache, block_table, ctx_lens, out, k_new, v_new)
        self.buckets = [int(b) for b in buckets]
        arr = (ctypes.c_int32 * len(self.buckets))(*self.buckets)
        handle = ctypes.c_void_p()
        none = AttnTensor(None, 0, 0, 0)
        s = stream if stream is not None else torch.cuda.Stream()
        self._stream = s
        st = lib.paged_decode_graphs_create(
            ctypes.byref(shape), arr, len(self.buckets), q.data_ptr(), q.stride(0), q.stride(1),
            _tensor(k_new, False) if k_new is not None else none, _tensor(v_new, False) if v_new is not None else none,
            AttnTensor(k_cache.data_ptr(), k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)),
            AttnTensor(v_cache.data_ptr(), v_cache.stride(0), v_cache.stride(1), v_cache.stride(2)),
            block_table.data_ptr(), ctx_lens.data_ptr(), scale, float(softcap), out.data_ptr(), out.stride(0),
            out.stride(1), self.workspace.data_ptr(), nbytes, s.cuda_stream, ctypes.byref(handle))
        _check(st, "paged_decode_graphs_create")
        self._handle = handle

    def launch(self, B: int) -> int:
        bucket = ctypes.c_int32(0)
        _check(load_library().paged_decode_graphs_launch(self._handle, int(B), _stream(), ctypes.byref(bucket)),
               "paged_decode_graphs_launch")
        return bucket.value

    def close(self) -> None:
        if self._handle is not None and self._handle.value:
            load_library().paged_decode_graphs_destroy(self._handle)
        self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _paged_shape(k_cache, block_table, B, D, dtype):
    num_pages, page_size, Hkv, Dc = k_cache.shape
    if Dc != D:
        raise ValueError("token rows and cache rows have different head_dim")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be (B, max_pages_per_seq), got {tuple(block_table.shape)}")
    return AttnDecodeShape(B, Hkv, Hkv, D, page_size, num_pages, block_table.shape[1], _DT16[dtype])


def _paged_checks(k_cache, v_cache, block_table, ctx_lens, B):
    _half(k_cache, "k_cache")
    _half(v_cache, "v_cache", k_cache.dtype)
    _expect(v_cache, tuple(k_cache.shape), "v_cache")
    for t, n in ((block_table, "block_table"), (ctx_lens, "ctx_lens")):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous int32 device tensor")
    _expect(ctx_lens, (B,), "ctx_lens")


def paged_kv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    block_table: torch.Tensor, ctx_lens: torch.Tensor) -> None:
    """Writes the n newest tokens k_new/v_new (B, n, Hkv, D) of each sequence into the paged caches
    (num_pages, page_size, Hkv, D): token i of sequence b goes to position ctx_lens[b] - n + i."""
    lib = load_library()
    B, n, Hkv, D = k_new.shape
    _paged_checks(k_cache, v_cache, block_table, ctx_lens, B)
    _half(k_new, "k_new", k_cache.dtype)
    _half(v_new, "v_new", k_cache.dtype)
    _expect(v_new, tuple(k_new.shape), "v_new")
    shape = _paged_shape(k_cache, block_table, B, D, k_cache.dtype)
    if Hkv != shape.Hkv:
        raise ValueError("token rows and cache rows have different kv head counts")
    st = lib.paged_kv_append(ctypes.byref(shape), n, _tensor(k_new, False), _tensor(v_new, False),
                             _tensor(k_cache, False), _tensor(v_cache, False), block_table.data_ptr(),
                             ctx_lens.data_ptr(), _stream())
    _check(st, "paged_kv_append")


def paged_kv_gather(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor, ctx_lens: torch.Tensor,
                    n_tokens: int, k_out: Optional[torch.Tensor] = None,
                    v_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The first n_tokens cached tokens of each sequence as contiguous (B, n_tokens, Hkv, D) K and V
    (zeros past ctx_lens[b])."""
    lib = load_library()
    B = block_table.shape[0]
    _, _, Hkv, D = k_cache.shape
    _paged_checks(k_cache, v_cache, block_table, ctx_lens, B)
    if k_out is None:
        k_out = torch.empty((B, n_tokens, Hkv, D), device=k_cache.device, dtype=k_cache.dtype)
    if v_out is None:
        v_out = torch.empty_like(k_out)
    for t, nm in ((k_out, "k_out"), (v_out, "v_out")):
        _half(t, nm, k_cache.dtype)
        _expect(t, (B, n_tokens, Hkv, D), nm)
    shape = _paged_shape(k_cache, block_table, B, D, k_cache.dtype)
    st = lib.paged_kv_gather(ctypes.byref(shape), int(n_tokens), _tensor(k_cache, False), _tensor(v_cache, False),
                             block_table.data_ptr(), ctx_lens.data_ptr(), _tensor(k_out, False),
                             _tensor(v_out, False), _stream())
    _check(st, "paged_kv_gather")
    return k_out, v_out


def _paged_fwd_args(q, k_cache, v_cache, block_table, cu_q, ctx_lens, max_q, scale, out, lse):
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _half(t, n, q.dtype)
    for t, n in ((block_table, "block_table"), (cu_q, "cu_q"), (ctx_lens, "ctx_lens")):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous int32 device tensor")
    T, Hq, D = q.shape
    B = cu_q.numel() - 1
    num_pages, page_size, Hkv, Dc = k_cache.shape
    if Dc != D:
        raise ValueError("k_cache head_dim differs from q's")
    _expect(v_cache, tuple(k_cache.shape), "v_cache")
    _expect(ctx_lens, (B,), "ctx_lens")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be (B, max_pages_per_seq), got {tuple(block_table.shape)}")
    shape = AttnPagedShape(B, int(max_q), T, Hq, Hkv, D, _DT16[q.dtype], page_size, num_pages, block_table.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((Hq, T), device=q.device, dtype=torch.float32) if lse is None else lse
    _half(out, "out", q.dtype)
    _expect(out, (T, Hq, D), "out")
    _expect(lse, (Hq, T), "lse")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    return shape, float(scale), out, lse


def attn_fwd_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                   cu_q: torch.Tensor, ctx_lens: torch.Tensor, max_q: int, scale: Optional[float] = None,
                   window: int = 0, softcap: float = 0.0, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O (T,Hq,D), LSE (Hq,T) of each sequence's new query rows q (T,Hq,D), packed by cu_q (B+1), against
    its paged cache (num_pages, page_size, Hkv, D) read through block_table (B, max_pages_per_seq);
    ctx_lens (B) counts the cached tokens, the new ones included (causal; see attn_fwd_paged)."""
    lib = load_library()
    shape, scale, out, lse = _paged_fwd_args(q, k_cache, v_cache, block_table, cu_q, ctx_lens, max_q, scale, out, lse)
    st = lib.attn_fwd_paged(ctypes.byref(shape), _tensor(q, True), _tensor(k_cache, False), _tensor(v_cache, False),
                            block_table.data_ptr(), cu_q.data_ptr(), ctx_lens.data_ptr(), scale, int(window),
                            float(softcap), _tensor(out, True), lse.data_ptr(), _stream())
    _check(st, "attn_fwd_paged")
    return out, lse


def attn_fwd_paged_workspace_bytes(q: torch.Tensor, k_cache: torch.Tensor, block_table: torch.Tensor,
                                   cu_q: torch.Tensor, max_q: int) -> int:
    """Workspace bytes attn_fwd_paged_split needs for these shapes (0 if it would refuse them)."""
    T, Hq, D = q.shape
    num_pages, page_size, Hkv, _ = k_cache.shape
    shape = AttnPagedShape(cu_q.numel() - 1, int(max_q), T, Hq, Hkv, D, _DT16.get(q.dtype, -1), page_size, num_pages,
                           block_table.shape[1])
    return int(load_library().attn_fwd_paged_workspace_bytes(ctypes.byref(shape)))


def attn_fwd_paged_split(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                         cu_q: torch.Tensor, ctx_lens: torch.Tensor, max_q: int, scale: Optional[float] = None,
                         window: int = 0, softcap: float = 0.0, out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """attn_fwd_paged with decode rows (sequences of one new token) split over several workgroups
    whose partial results a second kernel merges; workspace: a uint8 device tensor of at least
    attn_fwd_paged_workspace_bytes (allocated here when None)."""
    lib = load_library()
    shape, scale, out, lse = _paged_fwd_args(q, k_cache, v_cache, block_table, cu_q, ctx_lens, max_q, scale, out, lse)
    nbytes = int(lib.attn_fwd_paged_workspace_bytes(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.empty(nbytes, device=q.device, dtype=torch.uint8)
    st = lib.attn_fwd_paged_split(ctypes.byref(shape), _tensor(q, True), _tensor(k_cache, False),
                                  _tensor(v_cache, False), block_table.data_ptr(), cu_q.data_ptr(), ctx_lens.data_ptr(),
                                  scale, int(window), float(softcap), _tensor(out, True), lse.data_ptr(),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream())
    _check(st, "attn_fwd_paged_split")
    return out, lse


def debug(on: bool) -> bool:
    """Switches the library's metadata checks (debug mode) on or off; returns the previous mode."""
    return bool(load_library().attn_debug(1 if on else 0))


def count_restarts(counter: Optional[torch.Tensor]) -> None:
    """Forward kernels add their softmax-reference restarts to counter (a device int32 tensor of
    one element) until count_restarts(None)."""
    if counter is not None and (counter.dtype != torch.int32 or not counter.is_cuda):
        raise TypeError("counter must be an int32 device tensor")
    load_library().attn_count_restarts(counter.data_ptr() if counter is not None else None)


def peak_probe(kind: int, buf: torch.Tensor, reps: int = 1) -> None:
    """Launches roofline probe `kind` (0 matrix rate, 1 streaming read, 2 streaming copy) on the
    current stream over the device buffer buf (see attn_peak_probe)."""
    _check(load_library().attn_peak_probe(int(kind), buf.data_ptr(), buf.numel() * buf.element_size(), int(reps),
                                          _stream()), "attn_peak_probe")


def profile(on: bool) -> None:
    """Start / stop recording HIP event pairs around every kernel the library launches."""
    load_library().attn_profile(1 if on else 0)


def profile_read() -> dict:
    """{kernel name: (launches, total ms)} of the launches recorded since the last read."""
    lib = load_library()
    arr = (AttnKernelTime * 64)()
    n = lib.attn_profile_read(arr, 64)
    if n < 0:
        raise RuntimeError("attn_profile_read failed")
    return {arr[i].kernel.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n)}
