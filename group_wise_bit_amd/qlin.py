"""Python binding of libqlin (include/qlin.h): argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI.
PyTorch supplies device memory and the current stream.  There is no fallback:
if libqlin.so is missing or the GPU is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqlin.so")

FMT_PACKED = 0
FMT_FP16_MASTER = 1

STATUS_NAMES = {
    0: "QLIN_OK", 1: "QLIN_ERR_NULL", 2: "QLIN_ERR_SHAPE", 3: "QLIN_ERR_BITS",
    4: "QLIN_ERR_GROUP", 5: "QLIN_ERR_ALIGN", 6: "QLIN_ERR_FORMAT", 7: "QLIN_ERR_ALIAS",
    8: "QLIN_ERR_WORKSPACE", 9: "QLIN_ERR_NO_DEVICE", 10: "QLIN_ERR_HIP",
}

# Every symbol include/qlin.h declares.
EXPORTS = (
    "qlin_status_string", "qlin_last_hip_error", "qlin_abi_version", "qlin_packed_bytes",
    "qlin_meta_entries", "qlin_quantize", "qlin_gemv_workspace_bytes",
    "qlin_gemm_workspace_bytes", "qlin_gemv", "qlin_gemm",
    "qlin_gemv_multi_workspace_bytes", "qlin_gemv_multi",
    "qlin_gemv_swiglu_workspace_bytes", "qlin_gemv_swiglu", "qlin_embed_rows",
    "qlin_quantize_batch", "qlin_gemm_multi_workspace_bytes", "qlin_gemm_multi",
    "qlin_gemm_swiglu_workspace_bytes", "qlin_gemm_swiglu", "qlin_gemv_noalloc",
)
# include/qlin_tune.h (launch-shape sweeps and tests only)
TUNE_EXPORTS = ("qlin_set_launch_override",)
TUNE_FAMILIES = {"gemv": 0, "gemm": 1}


class QlinError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{where}: {_lib().qlin_status_string(status).decode()}"
        if hip_error:
            msg += f" (hip error {hip_error})"
        super().__init__(msg)


class QlinWeightC(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int32), ("k", ctypes.c_int32), ("bits", ctypes.c_int32),
        ("group", ctypes.c_int32), ("format", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("data", ctypes.c_void_p), ("ld", ctypes.c_int64),
        ("scale", ctypes.c_void_p), ("zero", ctypes.c_void_p),
    ]


class QlinQuantJobC(ctypes.Structure):
    _fields_ = [
        ("w16", ctypes.c_void_p), ("ld_w", ctypes.c_int64), ("n", ctypes.c_int32),
        ("k", ctypes.c_int32), ("codes", ctypes.c_void_p), ("scale", ctypes.c_void_p),
        ("zero", ctypes.c_void_p),
    ]


_LIB: Optional[ctypes.CDLL] = None


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libqlin.so not built at {LIB_PATH}; run "
                              "`python -m group_wise_bit_amd.build` (no CPU fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        wp = ctypes.POINTER(QlinWeightC)
        lib.qlin_status_string.argtypes = [ctypes.c_int]
        lib.qlin_status_string.restype = ctypes.c_char_p
        lib.qlin_last_hip_error.argtypes = []
        lib.qlin_last_hip_error.restype = ctypes.c_int
        lib.qlin_abi_version.argtypes = []
        lib.qlin_abi_version.restype = ctypes.c_int
        lib.qlin_packed_bytes.argtypes = [i32, i32, i32]
        lib.qlin_packed_bytes.restype = i64
        lib.qlin_meta_entries.argtypes = [i32, i32, i32]
        lib.qlin_meta_entries.restype = i64
        lib.qlin_quantize.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp]
        lib.qlin_quantize.restype = ctypes.c_int
        lib.qlin_gemv_workspace_bytes.argtypes = [wp]
        lib.qlin_gemv_workspace_bytes.restype = i64
        lib.qlin_gemm_workspace_bytes.argtypes = [wp, i32]
        lib.qlin_gemm_workspace_bytes.restype = i64
        lib.qlin_gemv.argtypes = [wp, vp, vp, vp, i64, vp]
        lib.qlin_gemv.restype = ctypes.c_int
        lib.qlin_gemm.argtypes = [wp, vp, i32, i64, vp, i64, vp, i64, vp]
        lib.qlin_gemm.restype = ctypes.c_int
        lib.qlin_gemv_multi_workspace_bytes.argtypes = [wp, i32]
        lib.qlin_gemv_multi_workspace_bytes.restype = i64
        lib.qlin_gemv_multi.argtypes = [wp, i32, vp, ctypes.POINTER(vp), vp, i64, vp]
        lib.qlin_gemv_multi.restype = ctypes.c_int
        lib.qlin_gemv_swiglu_workspace_bytes.argtypes = [wp]
        lib.qlin_gemv_swiglu_workspace_bytes.restype = i64
        lib.qlin_gemv_swiglu.argtypes = [wp, wp, vp, vp, vp, vp, i64, vp]
        lib.qlin_gemv_swiglu.restype = ctypes.c_int
        lib.qlin_embed_rows.argtypes = [wp, vp, i32, vp, vp, i64, vp]
        lib.qlin_embed_rows.restype = ctypes.c_int
        lib.qlin_quantize_batch.argtypes = [ctypes.POINTER(QlinQuantJobC), i32, i32, i32, vp]
        lib.qlin_quantize_batch.restype = ctypes.c_int
        lib.qlin_gemm_multi_workspace_bytes.argtypes = [wp, i32, i32]
        lib.qlin_gemm_multi_workspace_bytes.restype = i64
        lib.qlin_gemm_multi.argtypes = [wp, i32, vp, i32, i64, ctypes.POINTER(vp),
                                        ctypes.POINTER(i64), vp, i64, vp]
        lib.qlin_gemm_multi.restype = ctypes.c_int
        lib.qlin_gemm_swiglu_workspace_bytes.argtypes = [wp, i32]
        lib.qlin_gemm_swiglu_workspace_bytes.restype = i64
        lib.qlin_gemm_swiglu.argtypes = [wp, wp, vp, i32, i64, vp, vp, i64, vp, i64, vp]
        lib.qlin_gemm_swiglu.restype = ctypes.c_int
        lib.qlin_gemv_noalloc.argtypes = [wp, vp, vp, vp]
        lib.qlin_gemv_noalloc.restype = ctypes.c_int
        lib.qlin_set_launch_override.argtypes = [i32, ctypes.POINTER(i32)]
        lib.qlin_set_launch_override.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def library() -> ctypes.CDLL:
    """The loaded libqlin (raises ImportError when it is not built)."""
    return _lib()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise QlinError(status, where, _lib().qlin_last_hip_error() if status == 10 else 0)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need_out(t: torch.Tensor, dtype: torch.dtype, device: torch.device, rows: int, cols: int,
              name: str) -> None:
    """An output the library writes (it cannot see buffer sizes): the right
    dtype, on the inputs' device, unit-stride rows, room for rows x cols
    (rows = 0: a vector of cols elements)."""
    if not isinstance(t, torch.Tensor) or t.dtype != dtype:
        raise TypeError(f"{name} must be a {dtype} tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    if rows == 0:
        if not t.is_contiguous() or t.numel() < cols:
            raise ValueError(f"{name} must be contiguous with at least {cols} elements")
        return
    if t.dim() != 2 or t.stride(1) != 1 or t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name} must be 2-D [>= {rows}, >= {cols}] with contiguous rows, "
                         f"got shape {tuple(t.shape)} strides {t.stride()}")


def _need_x(w: "QWeight", x: torch.Tensor) -> None:
    if x.dtype != torch.float16 or x.numel() != w.k or not x.is_contiguous():
        raise TypeError(f"x must be a contiguous float16 tensor of k = {w.k} elements")


def set_launch_override(family: str, cfg=None) -> None:
    """qlin_set_launch_override (include/qlin_tune.h): force the launch shape of
    every later GEMV ("gemv": waves, splits[, rows]) or GEMM ("gemm": form,
    splits) call, or restore the library's own choice (cfg None).  cfg is a
    tuple or a "a,b[,c]" string.  For launch-shape sweeps and tests."""
    fam = TUNE_FAMILIES[family]
    if cfg is None:
        _check(_lib().qlin_set_launch_override(fam, None), "qlin_set_launch_override")
        return
    vals = [int(v) for v in cfg.split(",")] if isinstance(cfg, str) else [int(v) for v in cfg]
    if family == "gemv" and len(vals) == 2:
        vals.append(64)
    arr = (ctypes.c_int32 * 3)(*(vals + [0] * (3 - len(vals))))
    _check(_lib().qlin_set_launch_override(fam, arr), "qlin_set_launch_override")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def packed_bytes(n: int, k: int, bits: int) -> int:
    return int(_lib().qlin_packed_bytes(n, k, bits))


def meta_entries(n: int, k: int, group: int) -> int:
    return int(_lib().qlin_meta_entries(n, k, group))


@dataclass
class QWeight:
    """A weight matrix for qlin_gemv / qlin_gemm (tensors stay owned here)."""
    n: int
    k: int
    bits: int
    group: int
    format: int
    data: torch.Tensor
    scale: Optional[torch.Tensor] = None
    zero: Optional[torch.Tensor] = None
    ld: int = 0

    def c_struct(self) -> QlinWeightC:
        return QlinWeightC(self.n, self.k, self.bits, self.group, self.format, 0,
                           _ptr(self.data), self.ld, _ptr(self.scale), _ptr(self.zero))

    @property
    def weight_bytes(self) -> int:
        """Bytes a matmul must read for this weight (codes or fp16 + metadata)."""
        b = self.data.numel() * self.data.element_size() if self.format == FMT_PACKED \
            else self.n * self.k * 2
        if self.bits != 16:
            b += self.scale.numel() * 2 + self.zero.numel()
        return b


def _check_room(cbuf, code_bytes, scale, zero, entries) -> None:
    """The output buffers must hold what the library writes (it cannot check)."""
    if cbuf is not None and cbuf.numel() * cbuf.element_size() < code_bytes:
        raise ValueError(f"codes buffer holds {cbuf.numel() * cbuf.element_size()} bytes, "
                         f"{code_bytes} needed")
    if scale.numel() < entries or zero.numel() < entries:
        raise ValueError(f"scale/zero buffers hold fewer than {entries} entries")


def quantize(w16: torch.Tensor, bits: int, group: int, codes: bool = True,
             out: Optional[QWeight] = None) -> QWeight:
    """qlin_quantize on a cuda fp16 [n, k] tensor -> packed QWeight (codes=False:
    scale/zero only, returned with the masters as an FP16_MASTER weight)."""
    if w16.dtype != torch.float16 or w16.dim() != 2 or not w16.is_cuda:
        raise TypeError("w16 must be a 2-D cuda float16 tensor")
    if w16.stride(1) != 1:
        raise ValueError("w16 rows must be contiguous")
    n, k = w16.shape
    g = k if group in ("k", "K") else int(group)
    me = meta_entries(n, k, g)
    pb = packed_bytes(n, k, bits)
    if out is None:
        scale = torch.empty(max(me, 1), dtype=torch.float16, device=w16.device)
        zero = torch.empty(max(me, 1), dtype=torch.uint8, device=w16.device)
        cbuf = torch.empty(max(pb // 4, 1), dtype=torch.int32, device=w16.device) if codes else None
    else:
        scale, zero, cbuf = out.scale, out.zero, (out.data if codes else None)
    _check_room(cbuf, pb, scale, zero, me)
    st = _lib().qlin_quantize(w16.data_ptr(), w16.stride(0), n, k, bits, g, _ptr(cbuf),
                              scale.data_ptr(), zero.data_ptr(), _stream())
    _check(st, "qlin_quantize")
    if codes:
        return QWeight(n, k, bits, g, FMT_PACKED, cbuf, scale, zero)
    return QWeight(n, k, bits, g, FMT_FP16_MASTER, w16, scale, zero, ld=w16.stride(0))


def master_weight(w16: torch.Tensor, bits: int, group: int, scale=None, zero=None) -> QWeight:
    """FP16_MASTER weight over existing masters (bits=16: the plain fp16 control)."""
    n, k = w16.shape
    g = k if group in ("k", "K") else int(group)
    return QWeight(n, k, bits, g, FMT_FP16_MASTER, w16, scale, zero, ld=w16.stride(0))


_WS: dict = {}


def workspace(nbytes: int, device: torch.device) -> Optional[torch.Tensor]:
    """Zero-filled workspace, cached per (device, stream); the kernels leave it
    zero-filled again after every call."""
    if nbytes <= 0:
        return None
    key = (device.index, _stream())
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf


def gemv(w: QWeight, x: torch.Tensor, y: Optional[torch.Tensor] = None,
         ws: Optional[torch.Tensor] = "auto") -> torch.Tensor:
    _need_x(w, x)
    if y is None:
        y = torch.empty(w.n, dtype=torch.float32, device=x.device)
    _need_out(y, torch.float32, x.device, 0, w.n, "y")
    ws_struct = w.c_struct()
    if isinstance(ws, str):
        need = int(_lib().qlin_gemv_workspace_bytes(ctypes.byref(ws_struct)))
        ws = workspace(need, x.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = _lib().qlin_gemv(ctypes.byref(ws_struct), x.data_ptr(), y.data_ptr(), _ptr(ws), wsb,
                          _stream())
    _check(st, "qlin_gemv")
    return y


def gemv_noalloc(w: QWeight, x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """qlin_gemv_noalloc: qlin_gemv with the library's static split-K scratch
    (no workspace, no allocation inside the library; y is allocated here only
    when not given)."""
    _need_x(w, x)
    if y is None:
        y = torch.empty(w.n, dtype=torch.float32, device=x.device)
    _need_out(y, torch.float32, x.device, 0, w.n, "y")
    ws_struct = w.c_struct()
    st = _lib().qlin_gemv_noalloc(ctypes.byref(ws_struct), x.data_ptr(), y.data_ptr(), _stream())
    _check(st, "qlin_gemv_noalloc")
    return y


def gemm(w: QWeight, X: torch.Tensor, Y: Optional[torch.Tensor] = None,
         ws: Optional[torch.Tensor] = "auto") -> torch.Tensor:
    if X.dtype != torch.float16 or X.dim() != 2 or X.shape[1] != w.k or X.stride(1) != 1:
        raise TypeError("X must be a float16 [m, k] tensor with contiguous rows")
    m = X.shape[0]
    if Y is None:
        Y = torch.empty(m, w.n, dtype=torch.float32, device=X.device)
    _need_out(Y, torch.float32, X.device, m, w.n, "Y")
    ws_struct = w.c_struct()
    if isinstance(ws, str):
        need = int(_lib().qlin_gemm_workspace_bytes(ctypes.byref(ws_struct), m))
        ws = workspace(need, X.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = _lib().qlin_gemm(ctypes.byref(ws_struct), X.data_ptr(), m, X.stride(0), Y.data_ptr(),
                          Y.stride(0), _ptr(ws), wsb, _stream())
    _check(st, "qlin_gemm")
    return Y


def gemv_multi(ws_list: Sequence[QWeight], x: torch.Tensor,
               ys: Optional[Sequence[torch.Tensor]] = None,
               ws: Optional[torch.Tensor] = "auto") -> List[torch.Tensor]:
    """qlin_gemv_multi: y_i = W_i . x for up to 4 packed weights sharing x, one launch."""
    count = len(ws_list)
    for w in ws_list:
        _need_x(w, x)
    arr = (QlinWeightC * max(count, 1))(*[w.c_struct() for w in ws_list])
    if ys is None:
        ys = [torch.empty(w.n, dtype=torch.float32, device=x.device) for w in ws_list]
    if len(ys) != count:
        raise ValueError("one output per weight")
    for i, (w, y) in enumerate(zip(ws_list, ys)):
        _need_out(y, torch.float32, x.device, 0, w.n, f"ys[{i}]")
    yp = (ctypes.c_void_p * max(count, 1))(*[y.data_ptr() for y in ys])
    if isinstance(ws, str):
        need = int(_lib().qlin_gemv_multi_workspace_bytes(arr, count))
        ws = workspace(need, x.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = _lib().qlin_gemv_multi(arr, count, x.data_ptr(), yp, _ptr(ws), wsb, _stream())
    _check(st, "qlin_gemv_multi")
    return list(ys)


def gemv_swiglu(gate: QWeight, up: QWeight, x: torch.Tensor,
                h: Optional[torch.Tensor] = None, h16: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = "auto", want_h: bool = True,
                want_h16: bool = True) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """qlin_gemv_swiglu: h = silu(gate . x) * (up . x), fp32 and/or fp16, one launch."""
    _need_x(gate, x)
    _need_x(up, x)
    if h is None and want_h:
        h = torch.empty(gate.n, dtype=torch.float32, device=x.device)
    if h16 is None and want_h16:
        h16 = torch.empty(gate.n, dtype=torch.float16, device=x.device)
    if h is not None:
        _need_out(h, torch.float32, x.device, 0, gate.n, "h")
    if h16 is not None:
        _need_out(h16, torch.float16, x.device, 0, gate.n, "h16")
    g, u = gate.c_struct(), up.c_struct()
    if isinstance(ws, str):
        need = int(_lib().qlin_gemv_swiglu_workspace_bytes(ctypes.byref(g)))
        ws = workspace(need, x.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = _lib().qlin_gemv_swiglu(ctypes.byref(g), ctypes.byref(u), x.data_ptr(), _ptr(h),
                                 _ptr(h16), _ptr(ws), wsb, _stream())
    _check(st, "qlin_gemv_swiglu")
    return h, h16


def embed_rows(w: QWeight, ids: torch.Tensor, want16: bool = True, want32: bool = False
               ) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """qlin_embed_rows: dequantized rows ids of a packed weight, fp16 and/or fp32 [len(ids), k]."""
    if ids.dtype != torch.int32 or ids.dim() != 1 or not ids.is_contiguous():
        raise TypeError("ids must be a contiguous 1-D int32 tensor")
    count = ids.numel()
    out16 = torch.empty(count, w.k, dtype=torch.float16, device=ids.device) if want16 else None
    out32 = torch.empty(count, w.k, dtype=torch.float32, device=ids.device) if want32 else None
    ws_struct = w.c_struct()
    st = _lib().qlin_embed_rows(ctypes.byref(ws_struct), ids.data_ptr(), count, _ptr(out16),
                                _ptr(out32), w.k, _stream())
    _check(st, "qlin_embed_rows")
    return out16, out32


def quantize_batch(masters: Sequence[torch.Tensor], bits: int, group, codes: bool = True,
                   outs: Optional[Sequence[QWeight]] = None) -> List[QWeight]:
    """qlin_quantize_batch: every cuda fp16 [n, k] master quantized at one bit
    width, group 64 or "K" (per row), one launch per 64 matrices.  outs: the
    QWeights of an earlier call to overwrite (scale/zero, and codes)."""
    row = group in ("k", "K")
    if not row and int(group) != 64:
        raise ValueError("group must be 64 or 'K'")
    res, jobs = [], []
    for i, w16 in enumerate(masters):
        if w16.dtype != torch.float16 or w16.dim() != 2 or not w16.is_cuda or w16.stride(1) != 1:
            raise TypeError("masters must be 2-D cuda float16 tensors with contiguous rows")
        n, k = w16.shape
        g = k if row else 64
        me = meta_entries(n, k, g)
        if outs is not None:
            o = outs[i]
            scale, zero, cbuf = o.scale, o.zero, (o.data if codes else None)
            _check_room(cbuf, packed_bytes(n, k, bits), scale, zero, me)
        else:
            scale = torch.empty(max(me, 1), dtype=torch.float16, device=w16.device)
            zero = torch.empty(max(me, 1), dtype=torch.uint8, device=w16.device)
            cbuf = (torch.empty(max(packed_bytes(n, k, bits) // 4, 1), dtype=torch.int32,
                                device=w16.device) if codes else None)
        jobs.append(QlinQuantJobC(w16.data_ptr(), w16.stride(0), n, k, _ptr(cbuf),
                                  scale.data_ptr(), zero.data_ptr()))
        res.append(QWeight(n, k, bits, g, FMT_PACKED, cbuf, scale, zero) if codes else
                   QWeight(n, k, bits, g, FMT_FP16_MASTER, w16, scale, zero, ld=w16.stride(0)))
    arr = (QlinQuantJobC * max(len(jobs), 1))(*jobs)
    st = _lib().qlin_quantize_batch(arr, len(jobs), bits, 0 if row else 64, _stream())
    _check(st, "qlin_quantize_batch")
    return res


def gemm_multi(ws_list: Sequence[QWeight], X: torch.Tensor,
               Ys: Optional[Sequence[torch.Tensor]] = None,
               ws: Optional[torch.Tensor] = "auto") -> List[torch.Tensor]:
    """qlin_gemm_multi: Y_i = X . W_i^T for up to 4 packed weights sharing X, one launch."""
    if X.dtype != torch.float16 or X.dim() != 2 or X.stride(1) != 1:
        raise TypeError("X must be a float16 [m, k] tensor with contiguous rows")
    m, count = X.shape[0], len(ws_list)
    if Ys is None:
        Ys = [torch.empty(m, w.n, dtype=torch.float32, device=X.device) for w in ws_list]
    if len(Ys) != count:
        raise ValueError("one output per weight")
    for i, (w, Y) in enumerate(zip(ws_list, Ys)):
        if X.shape[1] != w.k:
            raise TypeError(f"X has {X.shape[1]} columns, weight {i} k = {w.k}")
        _need_out(Y, torch.float32, X.device, m, w.n, f"Ys[{i}]")
    arr = (QlinWeightC * max(count, 1))(*[w.c_struct() for w in ws_list])
    yp = (ctypes.c_void_p * max(count, 1))(*[y.data_ptr() for y in Ys])
    ld = (ctypes.c_int64 * max(count, 1))(*[y.stride(0) for y in Ys])
    if isinstance(ws, str):
        need = int(_lib().qlin_gemm_multi_workspace_bytes(arr, count, m))
        ws = workspace(need, X.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = _lib().qlin_gemm_multi(arr, count, X.data_ptr(), m, X.stride(0), yp, ld, _ptr(ws), wsb,
                                _stream())
    _check(st, "qlin_gemm_multi")
    return list(Ys)


def gemm_swiglu(gate: QWeight, up: QWeight, X: torch.Tensor,
                H: Optional[torch.Tensor] = None, H16: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = "auto", want_h: bool = True,
                want_h16: bool = True) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """qlin_gemm_swiglu: H = silu(X . gate^T) * (X . up^T), fp32 and/or fp16 [m, n], one launch.
    H and H16, when both given, must share one row stride."""
    if X.dtype != torch.float16 or X.dim() != 2 or X.stride(1) != 1:
        raise TypeError("X must be a float16 [m, k] tensor with contiguous rows")
    m = X.shape[0]
    if H is None and want_h:
        H = torch.empty(m, gate.n, dtype=torch.float32, device=X.device)
    if H16 is None and want_h16:
        H16 = torch.empty(m, gate.n, dtype=torch.float16, device=X.device)
    if X.shape[1] != gate.k or X.shape[1] != up.k:
        raise TypeError("X must have k columns")
    if H is not None:
        _need_out(H, torch.float32, X.device, m, gate.n, "H")
    if H16 is not None:
        _need_out(H16, torch.float16, X.device, m, gate.n, "H16")
    outs = [t for t in (H, H16) if t is not None]
    ld = outs[0].stride(0) if outs else gate.n
    if any(t.stride(0) != ld for t in outs):
        raise ValueError("H and H16 must share one row stride")
    g, u = gate.c_struct(), up.c_struct()
    if isinstance(ws, str):
        need = int(_lib().qlin_gemm_swiglu_workspace_bytes(ctypes.byref(g), m))
        ws = workspace(need, X.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = _lib().qlin_gemm_swiglu(ctypes.byref(g), ctypes.byref(u), X.data_ptr(), m, X.stride(0),
                                 _ptr(H), _ptr(H16), ld, _ptr(ws), wsb, _stream())
    _check(st, "qlin_gemm_swiglu")
    return H, H16
