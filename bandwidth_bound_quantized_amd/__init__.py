"""Python binding of libqgemv (ctypes): argument marshalling only.

Every step of the GEMV and the argmax runs in the HIP kernels of
libqgemv.so; this module checks dtypes/shapes/devices of torch tensors,
passes their device pointers and the current HIP stream to the C ABI, and
turns negative status codes into QgemvError. PyTorch only provides device
memory and streams. There is no fallback: if the library is missing the
import fails.

Build the library first: ``python bandwidth_bound_quantized_amd/build.py``
(or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")

BF16, INT8_G32, Q4_0_G32, INT4_G128, INT8_ROW, INT4_G64 = 0, 1, 2, 3, 4, 5
SRC_CANONICAL, SRC_BF16 = 0, 1
OK, EINVAL, ESHAPE, EALIGN, ERANGE, EHIP = 0, -1, -2, -3, -4, -5
MAX_BATCH = 8
FLAG_BATCH_INVARIANT = 1
ARGMAX_WS_WORDS_PER_ROW = 2
FUSED_ARGMAX_WS_WORDS_PER_ROW = 4096
GROUP = {BF16: 1, INT8_G32: 32, Q4_0_G32: 32, INT4_G128: 128, INT8_ROW: 0, INT4_G64: 64}   # 0: per row
FMT_NAMES = {BF16: "bf16", INT8_G32: "int8_g32", Q4_0_G32: "q4_0_g32", INT4_G128: "int4_g128",
             INT8_ROW: "int8_row", INT4_G64: "int4_g64"}


class QgemvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {_lib.qgemv_status_str(status).decode()}"
        if status == EHIP:
            msg += f" (hipError {_lib.qgemv_last_hip_error()})"
        super().__init__(msg)


def _load() -> ctypes.CDLL:
    # torch brings its own HIP runtime (soname libamdhip64.so.7). Loading it
    # first makes libqgemv bind to that same runtime; loading libqgemv first
    # would pull in a second HIP/HSA runtime and the two would fight over
    # the device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libqgemv.so not built at {LIB_PATH}; run "
                          "`python bandwidth_bound_quantized_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    c_i64, c_int, c_vp, c_sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    sig = {
        "qgemv_packed_size": (c_int, [c_int, c_i64, c_i64, ctypes.POINTER(c_sz), ctypes.POINTER(c_sz)]),
        "qgemv_pack": (c_int, [c_int, c_int, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp]),
        "qgemv_run": (c_int, [c_int, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_int, c_vp]),
        "qgemv_quantize": (c_int, [c_int, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp]),
        "qgemv_run_flags": (c_int, [c_int, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_int, c_int, c_vp]),
        "qgemv_run_fused": (c_int, [c_int, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_int, c_vp, c_vp]),
        "qgemv_run_grouped": (c_int, [c_vp, c_int, c_int, c_vp]),
        "qgemv_attention_workspace_size": (c_int, [c_int, c_int, c_int, c_int, c_i64, ctypes.POINTER(c_sz)]),
        "qgemv_attention_decode": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_i64,
                                           ctypes.c_float, c_vp, c_vp]),
        "qgemv_run_grouped_argmax": (c_int, [c_vp, c_int, c_int, c_int, c_vp, c_vp, c_vp]),
        "qgemv_grouped_class": (c_int, [c_int, c_i64, c_int]),
        "qgemv_argmax": (c_int, [c_vp, c_i64, c_int, c_vp, c_vp, c_vp]),
        "qgemv_argmax_noalloc": (c_int, [c_vp, c_i64, c_int, c_vp, c_vp]),
        "qgemv_stream_read": (c_int, [c_vp, c_sz, c_vp, c_int, c_int, c_vp]),
        "qgemv_status_str": (ctypes.c_char_p, [c_int]),
        "qgemv_last_hip_error": (c_int, []),
        "qgemv_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTS = ("qgemv_packed_size", "qgemv_pack", "qgemv_quantize", "qgemv_run", "qgemv_run_flags",
           "qgemv_run_fused", "qgemv_run_grouped", "qgemv_attention_workspace_size", "qgemv_attention_decode",
           "qgemv_run_grouped_argmax", "qgemv_grouped_class", "qgemv_argmax", "qgemv_argmax_noalloc",
           "qgemv_stream_read",
           "qgemv_status_str", "qgemv_last_hip_error", "qgemv_version")


def lib() -> ctypes.CDLL:
    return _lib


def version() -> str:
    return _lib.qgemv_version().decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise QgemvError(status, where)


# ------------------------------------------------------------------ host side
def packed_size(fmt: int, M: int, K: int) -> Tuple[int, int]:
    w = ctypes.c_size_t()
    s = ctypes.c_size_t()
    _check(_lib.qgemv_packed_size(fmt, M, K, ctypes.byref(w), ctypes.byref(s)), "qgemv_packed_size")
    return w.value, s.value


def pack(fmt: int, src_kind: int, src_w: np.ndarray, src_scales: Optional[np.ndarray], M: int,
         K: int) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Host arrays in, host arrays out (codes as uint8 bytes, scales as uint16 bits)."""
    wb, sb = packed_size(fmt, M, K)
    src_w = np.ascontiguousarray(src_w)
    dst_w = np.empty(wb, dtype=np.uint8)
    dst_s = np.empty(sb // 2, dtype=np.uint16) if sb else None
    sp = None
    if src_scales is not None:
        src_scales = np.ascontiguousarray(src_scales, dtype=np.uint16)
        sp = src_scales.ctypes.data
    st = _lib.qgemv_pack(fmt, src_kind, src_w.ctypes.data, sp, M, K, dst_w.ctypes.data,
                         dst_s.ctypes.data if dst_s is not None else None)
    _check(st, "qgemv_pack")
    return dst_w, dst_s


# ---------------------------------------------------------------- device side
def quantize(fmt: int, w, M: int, K: int, codes, scales, err=None, stream=None) -> None:
    """Device quantizer (qgemv_quantize): w bf16 bits [M][K] (int16/uint16/bfloat16), codes
    (uint8, packed_size's w_bytes), scales (int16/uint16, s_bytes / 2), err (int32 [1]) or None."""
    import torch
    wp = _dev_ptr(w, "w", (torch.int16, torch.uint16, torch.bfloat16))
    cp = _dev_ptr(codes, "codes")
    sp = _dev_ptr(scales, "scales", (torch.int16, torch.uint16))
    ep = _dev_ptr(err, "err", torch.int32) if err is not None else None
    wb, sb = packed_size(fmt, M, K)
    if w.numel() < M * K or codes.numel() * codes.element_size() < wb or scales.numel() * 2 < sb:
        raise ValueError("w, codes or scales too small for (fmt, M, K)")
    _check(_lib.qgemv_quantize(fmt, wp, M, K, cp, sp, ep, _stream_handle(stream)), "qgemv_quantize")


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev_ptr(t, what: str, dtype=None) -> int:
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{what} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def run(fmt: int, W, scales, x, y, M: int, K: int, batch: int, stream=None) -> None:
    """y[:batch, :M] = W x (float32), all device tensors; see qgemv.h for layouts.

    W: uint8 (any dtype works: only its bytes are read); scales: int16/uint16
    binary16 bits or None for bf16; x: bf16 bits (int16/uint16/bfloat16)
    [batch][K]; y: float32 [batch][M].
    """
    import torch
    wp = _dev_ptr(W, "W")
    sp = _dev_ptr(scales, "scales") if scales is not None else None
    xp = _dev_ptr(x, "x", (torch.int16, torch.uint16, torch.bfloat16))
    yp = _dev_ptr(y, "y", torch.float32)
    if y.numel() < batch * M or x.numel() < batch * K:
        raise ValueError("x or y too small for (batch, M, K)")
    st = _lib.qgemv_run(fmt, wp, sp, xp, yp, M, K, batch, _stream_handle(stream))
    _check(st, "qgemv_run")


def run_flags(fmt: int, W, scales, x, y, M: int, K: int, batch: int, flags: int, stream=None) -> None:
    """run() with qgemv_run_flags options (FLAG_BATCH_INVARIANT)."""
    import torch
    wp = _dev_ptr(W, "W")
    sp = _dev_ptr(scales, "scales") if scales is not None else None
    xp = _dev_ptr(x, "x", (torch.int16, torch.uint16, torch.bfloat16))
    yp = _dev_ptr(y, "y", torch.float32)
    if y.numel() < batch * M or x.numel() < batch * K:
        raise ValueError("x or y too small for (batch, M, K)")
    _check(_lib.qgemv_run_flags(fmt, wp, sp, xp, yp, M, K, batch, flags, _stream_handle(stream)),
           "qgemv_run_flags")


def run_ptr(fmt: int, wp: int, sp: Optional[int], xp: int, yp: int, M: int, K: int, batch: int,
            stream_handle: Optional[int]) -> None:
    """Raw-pointer form of run() for timing loops (no tensor checks)."""
    st = _lib.qgemv_run(fmt, wp, sp, xp, yp, M, K, batch, stream_handle)
    if st != OK:
        raise QgemvError(st, "qgemv_run")


def attention_workspace_size(batch: int, n_q: int, n_kv: int, head_dim: int, max_ctx: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.qgemv_attention_workspace_size(batch, n_q, n_kv, head_dim, max_ctx, ctypes.byref(n)),
           "qgemv_attention_workspace_size")
    return n.value


def attention_workspace(batch: int, n_q: int, n_kv: int, head_dim: int, max_ctx: int, device="cuda"):
    """A workspace for attention_decode (the splits' partial results; contents on entry do not matter)."""
    import torch
    n = attention_workspace_size(batch, n_q, n_kv, head_dim, max_ctx)
    return torch.empty((n + 15) // 16 * 4, dtype=torch.int32, device=device)


def attention_decode(q, k_cache, v_cache, ctx_lens, out, batch: int, n_q: int, n_kv: int, head_dim: int,
                     max_ctx: int, scale: float, ws, stream=None) -> None:
    """qgemv_attention_decode: grouped-query decode attention over a bf16 KV cache."""
    import torch
    qp = _dev_ptr(q, "q", torch.float32)
    kp = _dev_ptr(k_cache, "k_cache", (torch.int16, torch.uint16, torch.bfloat16))
    vp = _dev_ptr(v_cache, "v_cache", (torch.int16, torch.uint16, torch.bfloat16))
    lp = _dev_ptr(ctx_lens, "ctx_lens", torch.int32)
    op = _dev_ptr(out, "out", torch.float32)
    wp = _dev_ptr(ws, "ws")
    if (q.numel() < batch * n_q * head_dim or out.numel() < batch * n_q * head_dim
            or k_cache.numel() < batch * n_kv * max_ctx * head_dim or v_cache.numel() < batch * n_kv * max_ctx * head_dim
            or ctx_lens.numel() < batch
            or ws.numel() * ws.element_size() < attention_workspace_size(batch, n_q, n_kv, head_dim, max_ctx)):
        raise ValueError("a buffer is too small for the shape")
    _check(_lib.qgemv_attention_decode(qp, kp, vp, lp, op, batch, n_q, n_kv, head_dim, max_ctx, scale, wp,
                                       _stream_handle(stream)), "qgemv_attention_decode")


class Fusion(ctypes.Structure):
    """Mirror of qgemv_fusion (device pointers as integers; 0/None = unused)."""
    _fields_ = [("norm_input", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("residual", ctypes.c_void_p),
                ("swiglu_out", ctypes.c_void_p), ("argmax_idx", ctypes.c_void_p),
                ("argmax_ws", ctypes.c_void_p)]


def run_fused(fmt: int, W, scales, x, y, M: int, K: int, batch: int, *, norm_input=None,
              norm_weight=None, eps: float = 1e-5, residual=None, swiglu_out=None, argmax_idx=None,
              argmax_ws=None, stream=None) -> None:
    """qgemv_run_fused: the GEMV with RMSNorm of norm_input as its input (x None), a
    residual add or SwiGLU of paired rows in its epilogue, and optionally the argmax."""
    import torch
    f = Fusion()
    if norm_input is not None:
        f.norm_input = _dev_ptr(norm_input, "norm_input", torch.float32)
        f.norm_weight = _dev_ptr(norm_weight, "norm_weight", (torch.int16, torch.uint16, torch.bfloat16))
        if norm_input.numel() < batch * K or norm_weight.numel() < K:
            raise ValueError("norm_input or norm_weight too small")
    f.norm_eps = eps
    if residual is not None:
        f.residual = _dev_ptr(residual, "residual", torch.float32)
        if residual.numel() < batch * M:
            raise ValueError("residual too small")
    if swiglu_out is not None:
        f.swiglu_out = _dev_ptr(swiglu_out, "swiglu_out", (torch.int16, torch.uint16, torch.bfloat16))
        if swiglu_out.numel() < batch * (M // 2):
            raise ValueError("swiglu_out too small")
    if argmax_idx is not None:
        f.argmax_idx = _dev_ptr(argmax_idx, "argmax_idx", torch.int32)
        f.argmax_ws = _dev_ptr(argmax_ws, "argmax_ws", (torch.int64, torch.uint64))
        if argmax_ws.numel() < batch * FUSED_ARGMAX_WS_WORDS_PER_ROW or argmax_idx.numel() < batch:
            raise ValueError("argmax_ws or argmax_idx too small")
    wp = _dev_ptr(W, "W")
    sp = _dev_ptr(scales, "scales") if scales is not None else None
    xp = _dev_ptr(x, "x", (torch.int16, torch.uint16, torch.bfloat16)) if x is not None else None
    yp = _dev_ptr(y, "y", torch.float32) if y is not None else None
    if (x is not None and x.numel() < batch * K) or (y is not None and y.numel() < batch * M):
        raise ValueError("x or y too small for (batch, M, K)")
    _check(_lib.qgemv_run_fused(fmt, wp, sp, xp, yp, M, K, batch, ctypes.byref(f), _stream_handle(stream)),
           "qgemv_run_fused")


def run_fused_ptr(fmt: int, wp: int, sp: Optional[int], xp: Optional[int], yp: Optional[int], M: int, K: int,
                  batch: int, fusion: "Fusion", stream_handle) -> None:
    """Raw-pointer form of run_fused() for timing loops (no tensor checks)."""
    st = _lib.qgemv_run_fused(fmt, wp, sp, xp, yp, M, K, batch, ctypes.byref(fusion), stream_handle)
    if st != OK:
        raise QgemvError(st, "qgemv_run_fused")


class GemvDesc(ctypes.Structure):
    """Mirror of qgemv_gemv_desc."""
    _fields_ = [("W", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("fmt", ctypes.c_int32), ("M", ctypes.c_int32),
                ("K", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def grouped_descs(entries) -> "ctypes.Array":
    """entries: iterable of (fmt, W, scales, x, y, M, K) with device tensors (scales may be None)."""
    import torch
    items = list(entries)
    arr = (GemvDesc * len(items))()
    for i, (fmt, W, S, x, y, M, K) in enumerate(items):
        arr[i] = GemvDesc(_dev_ptr(W, "W"), _dev_ptr(S, "scales") if S is not None else None,
                          _dev_ptr(x, "x", (torch.int16, torch.uint16, torch.bfloat16)),
                          _dev_ptr(y, "y", torch.float32), fmt, M, K, 0)
    return arr


GROUP_ALONE, GROUP_XREG, GROUP_MFMA = 0, 1, 2


def grouped_class(fmt: int, K: int, batch: int) -> int:
    """Which launch qgemv_run_grouped gives a GEMV of this (fmt, K, batch):
    GROUP_XREG (one launch per format), GROUP_MFMA (one per format and K) or
    GROUP_ALONE (qgemv_grouped_class)."""
    st = _lib.qgemv_grouped_class(fmt, K, batch)
    if st < 0:
        raise QgemvError(st, "qgemv_grouped_class")
    return st


def run_grouped(descs, batch: int, stream=None) -> None:
    """Independent GEMVs in as few launches as possible (see qgemv_run_grouped)."""
    st = _lib.qgemv_run_grouped(ctypes.cast(descs, ctypes.c_void_p), len(descs), batch,
                                _stream_handle(stream))
    _check(st, "qgemv_run_grouped")


def run_grouped_ptr(descs, batch: int, stream_handle) -> None:
    st = _lib.qgemv_run_grouped(ctypes.cast(descs, ctypes.c_void_p), len(descs), batch, stream_handle)
    if st != OK:
        raise QgemvError(st, "qgemv_run_grouped")


def run_grouped_argmax(descs, batch: int, argmax_entry: int, ws, idx, stream=None) -> None:
    """run_grouped, then idx[:batch] = argmax of each row of descs[argmax_entry]'s y
    (fused into that GEMV's launch where the small-batch kernel computes it)."""
    import torch
    wsp = _dev_ptr(ws, "ws", (torch.int64, torch.uint64))
    ip = _dev_ptr(idx, "idx", torch.int32)
    if ws.numel() < batch * FUSED_ARGMAX_WS_WORDS_PER_ROW or idx.numel() < batch:
        raise ValueError("ws or idx too small")
    st = _lib.qgemv_run_grouped_argmax(ctypes.cast(descs, ctypes.c_void_p), len(descs), batch,
                                       argmax_entry, wsp, ip, _stream_handle(stream))
    _check(st, "qgemv_run_grouped_argmax")


def run_grouped_argmax_ptr(descs, batch: int, argmax_entry: int, wsp: int, ip: int, stream_handle) -> None:
    st = _lib.qgemv_run_grouped_argmax(ctypes.cast(descs, ctypes.c_void_p), len(descs), batch,
                                       argmax_entry, wsp, ip, stream_handle)
    if st != OK:
        raise QgemvError(st, "qgemv_run_grouped_argmax")


def fused_argmax_workspace(batch: int, device="cuda"):
    """A zero-filled workspace for run_grouped_argmax (left zero after every call)."""
    import torch
    return torch.zeros(batch * FUSED_ARGMAX_WS_WORDS_PER_ROW, dtype=torch.int64, device=device)


def argmax(logits, V: int, batch: int, ws, idx, stream=None) -> None:
    """idx[:batch] = first index of the max of each logits row (see qgemv.h)."""
    import torch
    lp = _dev_ptr(logits, "logits", torch.float32)
    wsp = _dev_ptr(ws, "ws", (torch.int64, torch.uint64))
    ip = _dev_ptr(idx, "idx", torch.int32)
    if ws.numel() < batch * ARGMAX_WS_WORDS_PER_ROW:
        raise ValueError("ws too small")
    st = _lib.qgemv_argmax(lp, V, batch, wsp, ip, _stream_handle(stream))
    _check(st, "qgemv_argmax")


def argmax_noalloc(logits, V: int, batch: int, idx, stream=None) -> None:
    """qgemv_argmax with the library's static per-device workspace (see qgemv.h)."""
    import torch
    lp = _dev_ptr(logits, "logits", torch.float32)
    ip = _dev_ptr(idx, "idx", torch.int32)
    st = _lib.qgemv_argmax_noalloc(lp, V, batch, ip, _stream_handle(stream))
    _check(st, "qgemv_argmax_noalloc")


def argmax_workspace(batch: int, device="cuda"):
    """A zero-filled argmax workspace (the kernel leaves it zero after every call)."""
    import torch
    return torch.zeros(batch * ARGMAX_WS_WORDS_PER_ROW, dtype=torch.int64, device=device)


def stream_read(buf, nbytes: int, sink, grid: int = 0, unroll: int = 4, stream=None) -> None:
    import torch
    bp = _dev_ptr(buf, "buf")
    sp = _dev_ptr(sink, "sink", (torch.int32, torch.uint32))
    st = _lib.qgemv_stream_read(bp, nbytes, sp, grid, unroll, _stream_handle(stream))
    _check(st, "qgemv_stream_read")
