"""Python binding of libbqd.so (the C ABI in include/bqd.h).

Argument marshalling only: every computation runs in the library's gfx950
kernels.  Functions take CUDA (HIP) torch tensors, check dtypes, shapes and
contiguity (the C ABI sees plain pointers, so buffer sizes are checked here,
before anything is launched), allocate missing outputs with torch, and pass
``torch.cuda.current_stream()`` unless a stream is given.  Any non-zero
status raises ``BQDError``.  If the library has not been built, every entry
point raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# BQD_LIB names another build of the same library (e.g. to compare two builds).
LIB_PATH = os.environ.get("BQD_LIB") or os.path.join(_HERE, "libbqd.so")

BQD_F32, BQD_F16 = 0, 1
BQD_SCALE_ROW_F32, BQD_SCALE_GROUP32_F16 = 0, 1
BQD_MAX_K = 65536
BQD_MAX_K_ANY = 2113664
BQD_MAX_TOKENS = 16
BQD_MAX_PROD_K = 32768
BQD_MAX_PASS_K = 24576
BQD_STATIC_PASS_BYTES = 16 << 20
BQD_INT8X_BLOCK = 512

ENTRY_POINTS = (
    "bqd_abi_version", "bqd_status_string", "bqd_init",
    "quantize_weights_int4_rowwise", "quantize_weights_int4_group32",
    "quantize_weights_int8_group32", "pack_int4_rows_host", "unpack_int4_rows_host",
    "quantize_act", "gemv_w4a8", "linear_w4a8", "gemv_w4a8_group32",
    "linear_w4a8_group32", "gemv_w8a16_group32", "gemm_w4a8_verify", "gemm_w4a8_verify_workspace_bytes",
    "layer_w4a8_forward",
    "decode_pass_desc_bytes", "decode_pass_encode", "decode_pass_w4a8", "decode_pass_w4a8_static",
    "read_probe", "gemv_w4a16", "add_rmsnorm_quant", "swiglu_quant", "linear_rmsnorm_w4a8",
    "quantize_weights_q6k", "gemv_q6k_f16", "int8x_counts_host", "int8x_stream_bytes_host",
    "int8x_encode_host", "gemv_int8x",
)


class BQDError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class LinearW4A8(C.Structure):
    """Mirror of ``bqd_linear_w4a8``."""
    _fields_ = [("wq", C.c_void_p), ("scales", C.c_void_p), ("bias", C.c_void_p),
                ("N", C.c_int32), ("K", C.c_int32), ("scale_kind", C.c_int32),
                ("r", C.c_int32), ("lanes_per_row", C.c_int32)]


_lib = None


def lib() -> C.CDLL:
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run "
                           "`python -m bit_quantized_decode_quantize_amd.csrc.build`")
    L = C.CDLL(LIB_PATH)
    P, I = C.c_void_p, C.c_int32
    sig = {
        "bqd_abi_version": (I, []),
        "bqd_status_string": (C.c_char_p, [I]),
        "bqd_init": (I, []),
        "quantize_weights_int4_rowwise": (I, [P, I, I, P, P, P]),
        "quantize_weights_int4_group32": (I, [P, I, I, P, P, P]),
        "quantize_weights_int8_group32": (I, [P, I, I, P, P, P]),
        "pack_int4_rows_host": (I, [P, I, I, P]),
        "unpack_int4_rows_host": (I, [P, I, I, P]),
        "quantize_act": (I, [P, I, I, I, P, P, P]),
        "gemv_w4a8": (I, [P, P, P, P, P, P, P, I, I, I, I, P]),
        "linear_w4a8": (I, [P, P, P, P, I, P, P, P, P, I, I, I, I, P]),
        "gemv_w4a8_group32": (I, [P, P, P, P, P, P, P, I, I, I, I, P]),
        "linear_w4a8_group32": (I, [P, P, P, P, I, P, P, P, P, I, I, I, I, P]),
        "gemv_w8a16_group32": (I, [P, P, P, P, I, I, I, I, P]),
        "gemm_w4a8_verify": (I, [P, P, P, P, P, P, P, I, I, I, I, P, C.c_size_t, P]),
        "gemm_w4a8_verify_workspace_bytes": (C.c_size_t, [I, I, I]),
        "layer_w4a8_forward": (I, [C.POINTER(LinearW4A8), I, P, I, P, P]),
        "decode_pass_desc_bytes": (C.c_size_t, [I]),
        "decode_pass_encode": (I, [C.POINTER(LinearW4A8), I, P, I, P, P, C.c_size_t, C.POINTER(C.c_int32),
                                   C.POINTER(C.c_size_t), C.POINTER(C.c_int32)]),
        "decode_pass_w4a8": (I, [P, I, I, I, P, C.c_size_t, I, P]),
        "decode_pass_w4a8_static": (I, [P, I, I, I, C.c_size_t, I, P, P]),
        "read_probe": (I, [P, C.c_size_t, P, I, I, P]),
        "gemv_w4a16": (I, [P, P, P, P, P, I, I, I, I, P]),
        "add_rmsnorm_quant": (I, [P, P, P, C.c_float, P, P, P, P, I, I, P]),
        "swiglu_quant": (I, [P, P, P, P, I, I, P]),
        "linear_rmsnorm_w4a8": (I, [P, P, P, P, P, P, C.c_float, P, P, P, P, P, I, I, I, I, P]),
        "quantize_weights_q6k": (I, [P, I, I, P, P, P, P, P]),
        "gemv_q6k_f16": (I, [P, P, P, P, P, P, I, I, I, I, P]),
        "int8x_counts_host": (I, [P, C.c_int64, P]),
        "int8x_stream_bytes_host": (I, [C.c_int64, P, P]),
        "int8x_encode_host": (I, [P, C.c_int64, P, P, P, P, P, P, P]),
        "gemv_int8x": (I, [P, P, P, P, P, P, P, P, P, P, C.c_float, P, P, I, I, I, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().bqd_status_string(status).decode()


def abi_version() -> int:
    return lib().bqd_abi_version()


def _call(name: str, *args) -> None:
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise BQDError(name, rc, status_string(rc))


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtypes, numel: Optional[int] = None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t


def _opt(t, name, dtypes, numel):
    return None if t is None else _dev(t, name, dtypes, numel)


def _empty(shape, dtype, like: torch.Tensor) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=like.device)


_WORD = (torch.int32,)
_F32 = (torch.float32,)
_X = (torch.float32, torch.float16)


def _xdtype(x: torch.Tensor) -> int:
    return BQD_F32 if x.dtype == torch.float32 else BQD_F16


# ---------------------------------------------------------------- weights --
def quantize_weights_int4_rowwise(W: torch.Tensor, wq=None, sw=None, stream=None):
    """W fp32 [N, K] -> (wq int32 [N, K/8] packed, sw fp32 [N])."""
    N, K = W.shape
    _dev(W, "W", _F32)
    wq = _empty((N, K // 8), torch.int32, W) if wq is None else _dev(wq, "wq", _WORD, N * K // 8)
    sw = _empty((N,), torch.float32, W) if sw is None else _dev(sw, "sw", _F32, N)
    _call("quantize_weights_int4_rowwise", W.data_ptr(), N, K, wq.data_ptr(), sw.data_ptr(),
          _stream(stream))
    return wq, sw


def quantize_weights_int4_group32(W: torch.Tensor, wq=None, s16=None, stream=None):
    """W fp32 [N, K] -> (wq int32 [N, K/8], s16 fp16 [N, K/32])."""
    N, K = W.shape
    _dev(W, "W", _F32)
    wq = _empty((N, K // 8), torch.int32, W) if wq is None else _dev(wq, "wq", _WORD, N * K // 8)
    s16 = _empty((N, K // 32), torch.float16, W) if s16 is None else \
        _dev(s16, "s16", (torch.float16,), N * (K // 32))
    _call("quantize_weights_int4_group32", W.data_ptr(), N, K, wq.data_ptr(), s16.data_ptr(),
          _stream(stream))
    return wq, s16


def quantize_weights_int8_group32(W: torch.Tensor, w8=None, s16=None, stream=None):
    """W fp32 [N, K] -> (w8 int8 [N, K] codes in [-32, 31], s16 fp16 [N, K/32])."""
    N, K = W.shape
    _dev(W, "W", _F32)
    w8 = _empty((N, K), torch.int8, W) if w8 is None else _dev(w8, "w8", (torch.int8,), N * K)
    s16 = _empty((N, K // 32), torch.float16, W) if s16 is None else \
        _dev(s16, "s16", (torch.float16,), N * (K // 32))
    _call("quantize_weights_int8_group32", W.data_ptr(), N, K, w8.data_ptr(), s16.data_ptr(),
          _stream(stream))
    return w8, s16


def pack_int4_rows_host(q: torch.Tensor) -> torch.Tensor:
    """Host: int8 codes [N, K] in [-8, 7] -> int32 words [N, K/8]."""
    q = q.detach().cpu().contiguous().to(torch.int8)
    N, K = q.shape
    out = torch.empty((N, K // 8), dtype=torch.int32)
    _call("pack_int4_rows_host", q.data_ptr(), N, K, out.data_ptr())
    return out


def unpack_int4_rows_host(w: torch.Tensor, K: Optional[int] = None) -> torch.Tensor:
    w = w.detach().cpu().contiguous().to(torch.int32)
    N = w.shape[0]
    K = w.shape[1] * 8 if K is None else K
    if w.numel() != N * K // 8:
        raise ValueError("word count does not match K")
    out = torch.empty((N, K), dtype=torch.int8)
    _call("unpack_int4_rows_host", w.data_ptr(), N, K, out.data_ptr())
    return out


# ------------------------------------------------------------ activations --
def quantize_act(x: torch.Tensor, qx=None, sx=None, stream=None):
    """x fp32/fp16 [K] or [M, K] -> (qx int8 like x, sx fp32 [M] (or [1]))."""
    _dev(x, "x", _X)
    x2 = x.view(1, -1) if x.dim() == 1 else x
    M, K = x2.shape
    qx = _empty(x.shape, torch.int8, x) if qx is None else _dev(qx, "qx", (torch.int8,), M * K)
    sx = _empty((M,), torch.float32, x) if sx is None else _dev(sx, "sx", _F32, M)
    _call("quantize_act", x.data_ptr(), _xdtype(x), M, K, qx.data_ptr(), sx.data_ptr(),
          _stream(stream))
    return qx, sx


def add_rmsnorm_quant(h, gamma, eps: float, delta=None, qx=None, sx=None, h_out=None, y_out=None,
                      quantize: bool = True, stream=None):
    """Residual add + RMSNorm + per-token quantisation of h fp32 [K] or [M, K]
    (delta: optional residual of the same shape; gamma fp32 [K]).  Returns
    (qx int8 like h, sx fp32 [M]); with quantize=False returns (None, None)
    and writes only the optional fp32 outputs h_out (h + delta) and y_out."""
    _dev(h, "h", _F32)
    h2 = h.view(1, -1) if h.dim() == 1 else h
    M, K = h2.shape
    _opt(delta, "delta", _F32, M * K)
    _dev(gamma, "gamma", _F32, K)
    _opt(h_out, "h_out", _F32, M * K)
    _opt(y_out, "y_out", _F32, M * K)
    if quantize:
        qx = _empty(h.shape, torch.int8, h) if qx is None else _dev(qx, "qx", (torch.int8,), M * K)
        sx = _empty((M,), torch.float32, h) if sx is None else _dev(sx, "sx", _F32, M)
    else:
        qx = sx = None
    _call("add_rmsnorm_quant", h.data_ptr(), _ptr(delta), gamma.data_ptr(), float(eps), _ptr(h_out),
          _ptr(y_out), _ptr(qx), _ptr(sx), M, K, _stream(stream))
    return qx, sx


def linear_rmsnorm_w4a8(wq, sw, bias, h, gamma, eps: float, delta=None, h_out=None, y=None,
                        want_q=False, want_acc=False, r=0, lanes_per_row=0, stream=None):
    """Residual add + RMSNorm + quantisation in the prologue of the W4A8
    linear: h, delta (optional), gamma fp32 [K]; h_out receives h + delta
    (must be another buffer).  Returns y, plus (qx, sx) if want_q, plus acc
    if want_acc."""
    N, K = _wshape(wq, None)
    _dev(wq, "wq", _WORD, N * K // 8)
    _dev(sw, "sw", _F32, N)
    _opt(bias, "bias", _F32, N)
    _dev(h, "h", _F32, K)
    _opt(delta, "delta", _F32, K)
    _dev(gamma, "gamma", _F32, K)
    _opt(h_out, "h_out", _F32, K)
    y = _empty((N,), torch.float32, wq) if y is None else _dev(y, "y", _F32, N)
    qx = _empty((K,), torch.int8, wq) if want_q else None
    sx = _empty((1,), torch.float32, wq) if want_q else None
    acc = _empty((N,), torch.int32, wq) if want_acc else None
    _call("linear_rmsnorm_w4a8", wq.data_ptr(), sw.data_ptr(), _ptr(bias), h.data_ptr(), _ptr(delta),
          gamma.data_ptr(), float(eps), _ptr(h_out), y.data_ptr(), _ptr(qx), _ptr(sx), _ptr(acc), N, K, r,
          lanes_per_row, _stream(stream))
    out = [y]
    if want_q:
        out += [qx, sx]
    if want_acc:
        out.append(acc)
    return out[0] if len(out) == 1 else tuple(out)


def swiglu_quant(gu, qx=None, sx=None, h_out=None, quantize: bool = True, stream=None):
    """SwiGLU of the fused gate/up output gu fp32 [2I] or [M, 2I] (gate, then
    up) + per-token quantisation.  h_out (fp32 [M, I]) receives h and is
    allocated when not given.  Returns (qx int8 [M, I] (or [I]), sx fp32
    [M]); with quantize=False returns (None, None) and writes only h_out."""
    _dev(gu, "gu", _F32)
    g2 = gu.view(1, -1) if gu.dim() == 1 else gu
    M, I2 = g2.shape
    if I2 % 2:
        raise ValueError("gu must hold 2I values per token")
    I_ = I2 // 2
    h_out = _empty((M, I_), torch.float32, gu) if h_out is None else _dev(h_out, "h_out", _F32, M * I_)
    shape = (I_,) if gu.dim() == 1 else (M, I_)
    if quantize:
        qx = _empty(shape, torch.int8, gu) if qx is None else _dev(qx, "qx", (torch.int8,), M * I_)
        sx = _empty((M,), torch.float32, gu) if sx is None else _dev(sx, "sx", _F32, M)
    else:
        qx = sx = None
    _call("swiglu_quant", gu.data_ptr(), _ptr(h_out), _ptr(qx), _ptr(sx), M, I_, _stream(stream))
    return qx, sx


# ------------------------------------------------------------------ GEMVs --
def _wshape(wq: torch.Tensor, K: Optional[int]):
    N = wq.shape[0]
    K = wq.shape[1] * 8 if K is None else K
    return N, K


def gemv_w4a8(wq, sw, bias, qx, sx, y=None, acc=None, r=0, lanes_per_row=0, stream=None):
    """y[j] = sw[j]*sx*acc[j] + b[j] over packed per-row INT4 weights and int8 qx.
    ``acc=True`` also returns the int32 accumulators."""
    N, K = _wshape(wq, None)
    _dev(wq, "wq", _WORD, N * K // 8)
    _dev(sw, "sw", _F32, N)
    _opt(bias, "bias", _F32, N)
    _dev(qx, "qx", (torch.int8,), K)
    _dev(sx, "sx", _F32)
    if sx.numel() < 1:
        raise ValueError("sx must hold one value")
    y = _empty((N,), torch.float32, wq) if y is None else _dev(y, "y", _F32, N)
    want = acc is True
    acc_t = _empty((N,), torch.int32, wq) if want else _opt(acc if acc is not False else None,
                                                            "acc", (torch.int32,), N)
    _call("gemv_w4a8", wq.data_ptr(), sw.data_ptr(), _ptr(bias), qx.data_ptr(), sx.data_ptr(),
          y.data_ptr(), _ptr(acc_t), N, K, r, lanes_per_row, _stream(stream))
    return (y, acc_t) if acc_t is not None else y


def linear_w4a8(wq, sw, bias, x, y=None, want_q=False, want_acc=False, r=0, lanes_per_row=0,
                stream=None):
    """Quantise x (fp32/fp16 [K]) in the GEMV prologue, then the W4A8 GEMV.
    Returns y, plus (qx, sx) if want_q, plus acc if want_acc."""
    N, K = _wshape(wq, None)
    _dev(wq, "wq", _WORD, N * K // 8)
    _dev(sw, "sw", _F32, N)
    _opt(bias, "bias", _F32, N)
    _dev(x, "x", _X, K)
    y = _empty((N,), torch.float32, wq) if y is None else _dev(y, "y", _F32, N)
    qx = _empty((K,), torch.int8, wq) if want_q else None
    sx = _empty((1,), torch.float32, wq) if want_q else None
    acc = _empty((N,), torch.int32, wq) if want_acc else None
    _call("linear_w4a8", wq.data_ptr(), sw.data_ptr(), _ptr(bias), x.data_ptr(), _xdtype(x),
          y.data_ptr(), _ptr(qx), _ptr(sx), _ptr(acc), N, K, r, lanes_per_row, _stream(stream))
    out = [y]
    if want_q:
        out += [qx, sx]
    if want_acc:
        out.append(acc)
    return out[0] if len(out) == 1 else tuple(out)


def gemv_w4a8_group32(wq, s16, bias, qx, sx, y=None, acc_g=None, r=0, lanes_per_row=0,
                      stream=None):
    """Group-32 W4A8: y = sx * sum_g s_g acc_g + b.  ``acc_g=True`` also
    returns the int32 per-group partials [N, K/32]."""
    N, K = _wshape(wq, None)
    _dev(wq, "wq", _WORD, N * K // 8)
    _dev(s16, "s16", (torch.float16,), N * (K // 32))
    _opt(bias, "bias", _F32, N)
    _dev(qx, "qx", (torch.int8,), K)
    _dev(sx, "sx", _F32)
    y = _empty((N,), torch.float32, wq) if y is None else _dev(y, "y", _F32, N)
    accg = _empty((N, K // 32), torch.int32, wq) if acc_g is True else None
    _call("gemv_w4a8_group32", wq.data_ptr(), s16.data_ptr(), _ptr(bias), qx.data_ptr(),
          sx.data_ptr(), y.data_ptr(), _ptr(accg), N, K, r, lanes_per_row, _stream(stream))
    return (y, accg) if accg is not None else y


def linear_w4a8_group32(wq, s16, bias, x, y=None, want_q=False, want_acc=False, r=0,
                        lanes_per_row=0, stream=None):
    N, K = _wshape(wq, None)
    _dev(wq, "wq", _WORD, N * K // 8)
    _dev(s16, "s16", (torch.float16,), N * (K // 32))
    _opt(bias, "bias", _F32, N)
    _dev(x, "x", _X, K)
    y = _empty((N,), torch.float32, wq) if y is None else _dev(y, "y", _F32, N)
    qx = _empty((K,), torch.int8, wq) if want_q else None
    sx = _empty((1,), torch.float32, wq) if want_q else None
    accg = _empty((N, K // 32), torch.int32, wq) if want_acc else None
    _call("linear_w4a8_group32", wq.data_ptr(), s16.data_ptr(), _ptr(bias), x.data_ptr(),
          _xdtype(x), y.data_ptr(), _ptr(qx), _ptr(sx), _ptr(accg), N, K, r, lanes_per_row,
          _stream(stream))
    out = [y]
    if want_q:
        out += [qx, sx]
    if want_acc:
        out.append(accg)
    return out[0] if len(out) == 1 else tuple(out)


def gemv_w8a16_group32(w8, s16, x16, y=None, r=0, lanes_per_row=0, stream=None):
    """int8 codes [N, K] x fp16 group-32 scales against fp16 x [K] -> fp32 y [N]."""
    N, K = w8.shape
    _dev(w8, "w8", (torch.int8,), N * K)
    _dev(s16, "s16", (torch.float16,), N * (K // 32))
    _dev(x16, "x16", (torch.float16,), K)
    y = _empty((N,), torch.float32, w8) if y is None else _dev(y, "y", _F32, N)
    _call("gemv_w8a16_group32", w8.data_ptr(), s16.data_ptr(), x16.data_ptr(), y.data_ptr(), N, K,
          r, lanes_per_row, _stream(stream))
    return y


class Q6KWeights:
    """Packed 6-bit weights: ql uint8 [N, K/2], qh uint8 [N, K/4], sc int8
    [N, K/16], d fp16 [N, K/256] (the layout of ``quantize_weights_q6k``)."""

    def __init__(self, ql, qh, sc, d):
        self.ql, self.qh, self.sc, self.d = ql, qh, sc, d
        self.N, self.K = ql.shape[0], ql.shape[1] * 2

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.ql, self.qh, self.sc, self.d))


def quantize_weights_q6k(W: torch.Tensor, stream=None) -> Q6KWeights:
    """fp32 W [N, K] (K % 256 == 0) on the device -> packed 6-bit weights."""
    _dev(W, "W", _F32)
    N, K = W.shape
    ql = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    qh = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    sc = torch.empty((N, K // 16), dtype=torch.int8, device=W.device)
    d = torch.empty((N, K // 256), dtype=torch.float16, device=W.device)
    _call("quantize_weights_q6k", W.data_ptr(), N, K, ql.data_ptr(), qh.data_ptr(), sc.data_ptr(),
          d.data_ptr(), _stream(stream))
    return Q6KWeights(ql, qh, sc, d)


def gemv_q6k_f16(w: Q6KWeights, x16, y=None, r=0, lanes_per_row=0, stream=None):
    """Packed 6-bit weights against fp16 x [K] -> fp32 y [N]."""
    N, K = w.N, w.K
    _dev(w.ql, "ql", (torch.uint8,), N * K // 2)
    _dev(w.qh, "qh", (torch.uint8,), N * K // 4)
    _dev(w.sc, "sc", (torch.int8,), N * K // 16)
    _dev(w.d, "d", (torch.float16,), N * K // 256)
    _dev(x16, "x16", (torch.float16,), K)
    y = _empty((N,), torch.float32, w.ql) if y is None else _dev(y, "y", _F32, N)
    _call("gemv_q6k_f16", w.ql.data_ptr(), w.qh.data_ptr(), w.sc.data_ptr(), w.d.data_ptr(), x16.data_ptr(),
          y.data_ptr(), N, K, r, lanes_per_row, _stream(stream))
    return y


INT8X_ARRAYS = ("b1", "b2", "l1", "l2", "l3", "b1_blk", "b2_blk")


class Int8XWeights:
    """INT8-X (3,5,8) encoded weights [N, K] on the device: the seven arrays,
    their byte sizes, the level counts and the per-tensor scale."""

    def __init__(self, arrays: dict, sizes, counts, N: int, K: int, sw: float):
        self.arrays, self.sizes, self.counts = arrays, sizes, counts
        self.N, self.K, self.sw = N, K, float(sw)
        self._sizes_c = (C.c_int64 * 7)(*sizes)

    def payload_bits(self) -> int:
        n1, n2, n3 = self.counts
        n = self.N * self.K
        return n + n2 + n3 + 3 * n1 + 5 * n2 + 8 * n3

    def nbytes(self) -> int:
        return int(sum(self.sizes))


def int8x_encode(q: torch.Tensor, sw: float, device="cuda") -> Int8XWeights:
    """Encode host int8 codes q [N, K] (the offline step of section 2.5) and
    upload the arrays to ``device``."""
    if q.dtype != torch.int8 or q.dim() != 2:
        raise TypeError("q must be a 2-D int8 tensor")
    q = q.detach().cpu().contiguous()
    N, K = q.shape
    n = N * K
    counts = (C.c_int64 * 3)()
    _call("int8x_counts_host", q.data_ptr(), n, counts)
    sizes = (C.c_int64 * 7)()
    _call("int8x_stream_bytes_host", n, counts, sizes)
    host = {}
    for name, nb in zip(INT8X_ARRAYS, sizes):
        dt = torch.uint8 if name == "l3" else torch.int32
        host[name] = torch.zeros(nb // (1 if dt == torch.uint8 else 4), dtype=dt)
    _call("int8x_encode_host", q.data_ptr(), n, *[host[k].data_ptr() for k in INT8X_ARRAYS])
    dev = {k: v.to(device) for k, v in host.items()}
    return Int8XWeights(dev, list(sizes), tuple(counts), N, K, sw)


def gemv_int8x(w: Int8XWeights, qx, sx, y=None, acc=None, rows=0, stream=None):
    """W8A8 GEMV over INT8-X weights: qx int8 [K], sx fp32 [1] -> y fp32 [N]
    (and acc int32 [N] with acc=True)."""
    _dev(qx, "qx", (torch.int8,), w.K)
    _dev(sx, "sx", _F32)
    a = w.arrays
    y = _empty((w.N,), torch.float32, qx) if y is None else _dev(y, "y", _F32, w.N)
    acc_t = _empty((w.N,), torch.int32, qx) if acc is True else None
    _call("gemv_int8x", *[a[k].data_ptr() for k in INT8X_ARRAYS], w._sizes_c, qx.data_ptr(), sx.data_ptr(),
          w.sw, y.data_ptr(), _ptr(acc_t), w.N, w.K, rows, _stream(stream))
    return (y, acc_t) if acc_t is not None else y


def gemv_w4a16(wq, sw, bias, x16, y=None, r=0, lanes_per_row=0, stream=None):
    """W4A16 comparison GEMV: packed per-row INT4 weights against fp16 x [K]
    (unpacked to fp16, fp32 accumulation) -> fp32 y [N]."""
    N, K = _wshape(wq, None)
    _dev(wq, "wq", _WORD, N * K // 8)
    _dev(sw, "sw", _F32, N)
    _opt(bias, "bias", _F32, N)
    _dev(x16, "x16", (torch.float16,), K)
    y = _empty((N,), torch.float32, wq) if y is None else _dev(y, "y", _F32, N)
    _call("gemv_w4a16", wq.data_ptr(), sw.data_ptr(), _ptr(bias), x16.data_ptr(), y.data_ptr(), N, K, r,
          lanes_per_row, _stream(stream))
    return y


_VERIFY_WS = {}


def verify_workspace(M: int, N: int, K: int, device) -> Optional[torch.Tensor]:
    """A zero-filled workspace of at least the bytes gemm_w4a8_verify needs
    for this shape, kept per device and grown when a shape needs more (the
    kernel leaves it zeroed).  None when the shape needs none.  Calls that
    share it must not overlap in time (one stream)."""
    nb = lib().gemm_w4a8_verify_workspace_bytes(M, N, K)
    if nb == 0:
        return None
    dev = torch.device(device)
    key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
    ws = _VERIFY_WS.get(key)
    if ws is None or ws.numel() * 4 < nb:
        ws = torch.zeros((nb + 255) // 4, dtype=torch.int32, device=dev)
        _VERIFY_WS[key] = ws
    return ws


def gemm_w4a8_verify(wq, sw, bias, qx, sx, y=None, acc=None, impl=0, workspace=None, stream=None):
    """M tokens: qx int8 [M, K], sx fp32 [M] -> y fp32 [M, N] (and acc [M, N]).
    ``workspace``: int32 device tensor for the balanced matrix-core kernel
    (default: ``verify_workspace``'s shared one)."""
    N, K = _wshape(wq, None)
    M = qx.shape[0]
    _dev(wq, "wq", _WORD, N * K // 8)
    _dev(sw, "sw", _F32, N)
    _opt(bias, "bias", _F32, N)
    _dev(qx, "qx", (torch.int8,), M * K)
    _dev(sx, "sx", _F32, M)
    y = _empty((M, N), torch.float32, wq) if y is None else _dev(y, "y", _F32, M * N)
    acc_t = _empty((M, N), torch.int32, wq) if acc is True else None
    if workspace is None and M >= 1 and N >= 1:
        workspace = verify_workspace(M, N, K, wq.device)
    if workspace is not None:
        _dev(workspace, "workspace", (torch.int32,))
    _call("gemm_w4a8_verify", wq.data_ptr(), sw.data_ptr(), _ptr(bias), qx.data_ptr(),
          sx.data_ptr(), y.data_ptr(), _ptr(acc_t), M, N, K, impl, _ptr(workspace),
          0 if workspace is None else workspace.numel() * 4, _stream(stream))
    return (y, acc_t) if acc_t is not None else y


def make_linear(wq, scales, bias=None, r=0, lanes_per_row=0) -> LinearW4A8:
    """Descriptor of one linear for layer_w4a8_forward / DecodePass.  The
    descriptor holds references to its tensors (``_tensors``), and LayerPlan
    and DecodePass hold their descriptors, so the device memory they point
    to stays allocated while they exist (the C structure itself carries only
    raw pointers)."""
    N, K = _wshape(wq, None)
    _dev(wq, "wq", _WORD, N * K // 8)
    if scales.dtype == torch.float32:
        _dev(scales, "scales", _F32, N)
        kind = BQD_SCALE_ROW_F32
    else:
        _dev(scales, "scales", (torch.float16,), N * (K // 32))
        kind = BQD_SCALE_GROUP32_F16
    _opt(bias, "bias", _F32, N)
    d = LinearW4A8(wq.data_ptr(), scales.data_ptr(), _ptr(bias), N, K, kind, r, lanes_per_row)
    d._tensors = (wq, scales, bias)
    return d


class LayerPlan:
    """Host-side arrays for layer_w4a8_forward, built once and replayed."""

    def __init__(self, linears: Sequence[LinearW4A8], xs: Sequence[torch.Tensor],
                 ys: Sequence[torch.Tensor]):
        n = len(linears)
        if not (len(xs) == len(ys) == n):
            raise ValueError("one x and one y per linear")
        dt = xs[0].dtype if n else torch.float32
        for i, (l, x, y) in enumerate(zip(linears, xs, ys)):
            _dev(x, f"x[{i}]", (dt,), l.K)
            _dev(y, f"y[{i}]", _F32, l.N)
        self.n = n
        self.x_dtype = BQD_F32 if dt == torch.float32 else BQD_F16
        self.lin = (LinearW4A8 * max(n, 1))(*linears)
        self.xp = (C.c_void_p * max(n, 1))(*[x.data_ptr() for x in xs])
        self.yp = (C.c_void_p * max(n, 1))(*[y.data_ptr() for y in ys])
        self._keep = (list(xs), list(ys), list(linears))

    def run(self, stream=None):
        _call("layer_w4a8_forward", self.lin, self.n, C.cast(self.xp, C.c_void_p), self.x_dtype,
              C.cast(self.yp, C.c_void_p), _stream(stream))


def layer_w4a8_forward(linears: Sequence[LinearW4A8], xs: Sequence[torch.Tensor],
                       ys: Sequence[torch.Tensor], stream=None) -> None:
    """Run the linears of one layer in order (one fused launch each)."""
    LayerPlan(linears, xs, ys).run(stream)


class DecodePass:
    """One persistent launch per decode step over ``linears`` in order
    (decode_pass_w4a8).  Encodes the descriptors once on the host, keeps a
    device copy and the zero-initialised workspace (error word, epoch words
    and the exchange through which linears read earlier outputs)."""

    def __init__(self, linears: Sequence[LinearW4A8], xs: Sequence[torch.Tensor],
                 ys: Sequence[torch.Tensor], device=None):
        n = len(linears)
        if n == 0:
            raise ValueError("a pass needs at least one linear")
        dt = xs[0].dtype
        for i, (l, x, y) in enumerate(zip(linears, xs, ys)):
            _dev(x, f"x[{i}]", (dt,), l.K)
            _dev(y, f"y[{i}]", _F32, l.N)
        device = xs[0].device if device is None else device
        self.n = n
        lin = (LinearW4A8 * n)(*linears)
        xp = (C.c_void_p * n)(*[x.data_ptr() for x in xs])
        yp = (C.c_void_p * n)(*[y.data_ptr() for y in ys])
        nbytes = lib().decode_pass_desc_bytes(n)
        host = (C.c_uint8 * nbytes)()
        mk = C.c_int32(0)
        sb = C.c_size_t(0)
        sl = C.c_int32(0)
        _call("decode_pass_encode", lin, n, C.cast(xp, C.c_void_p), BQD_F32 if dt == torch.float32 else BQD_F16,
              C.cast(yp, C.c_void_p), C.cast(host, C.c_void_p), nbytes, C.byref(mk), C.byref(sb), C.byref(sl))
        self.max_k = mk.value
        self.sync_bytes = sb.value
        self.slots = sl.value  # chunks per lane per step: the kernel instance
        self.desc = torch.frombuffer(bytearray(host), dtype=torch.uint8).to(device)
        self.sync = torch.zeros(self.sync_bytes // 4, dtype=torch.int32, device=device)
        self._keep = (list(xs), list(ys), list(linears))

    def run(self, stream=None, spin_limit: int = 0) -> None:
        _call("decode_pass_w4a8", self.desc.data_ptr(), self.n, self.max_k, self.slots, self.sync.data_ptr(),
              self.sync_bytes, spin_limit, _stream(stream))

    def run_static(self, err: torch.Tensor, stream=None, spin_limit: int = 0) -> None:
        """The same pass over the library's static per-GPU workspace
        (decode_pass_w4a8_static): allocates nothing; the error word lands in
        ``err`` (one int32 on the device)."""
        _dev(err, "err", (torch.int32,), 1)
        _call("decode_pass_w4a8_static", self.desc.data_ptr(), self.n, self.max_k, self.slots, self.sync_bytes,
              spin_limit, err.data_ptr(), _stream(stream))

    def error_word(self) -> int:
        """Bit 0: a wait ran out of spins; bit 1: descriptors for another
        grid (synchronises)."""
        return int(self.sync[0].item())

    def clear_error(self) -> None:
        self.sync[0].zero_()

    def sources(self) -> List[int]:
        """Per linear, the exchange word its activation starts at (>= 0: the
        activation is an earlier output of the pass), or -1 (written before
        the launch); read back from the encoded descriptors."""
        raw = self.desc.cpu().numpy().tobytes()
        return [int.from_bytes(raw[DESC_HEADER + DESC_TASK * i + 76:DESC_HEADER + DESC_TASK * i + 80], "little",
                               signed=True) for i in range(self.n)]


DESC_HEADER, DESC_TASK = 32, 96   # bytes of the descriptor header and of one linear's descriptor


def read_probe(buf: torch.Tensor, sink: torch.Tensor, grid: int, unroll: int = 1, stream=None) -> None:
    """Streaming read of ``buf`` (the read-ceiling reference kernel); ``sink``
    int32/uint32 with at least ``grid`` elements."""
    _dev(buf, "buf", (buf.dtype,))
    _dev(sink, "sink", (torch.int32,))
    if sink.numel() < grid:
        raise ValueError(f"sink holds {sink.numel()} words, the grid needs {grid}")
    _call("read_probe", buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), grid, unroll,
          _stream(stream))
