"""ctypes front end of the C oracle (oracle.c).

TEST INFRASTRUCTURE: imported only by tests/, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of bench.py.  Arrays are numpy; every function copies
its inputs to C-contiguous arrays of the documented dtype and returns new
numpy arrays.  Errors from the C side raise ``OracleError``.

Pages cited (by title and section):
  [Orin]   "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到 24 tok/s"
  [Ascend] "在香橙派上跑 Gemma4：vLLM 适配昇腾 310B 的内核开发实录"
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("BQD_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_ERR = {-1: "bad argument", -2: "value outside the format's range",
        -3: "non-finite input", -4: "accumulator outside the int32 bound"}


class OracleError(RuntimeError):
    pass


def _load():
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = C.CDLL(_LIB_PATH)
    P, I64, I32, F32 = C.c_void_p, C.c_int64, C.c_int, C.c_float
    sig = {
        "orc_f16_to_f32": (C.c_float, [C.c_uint16]),
        "orc_f32_to_f16": (C.c_uint16, [C.c_float]),
        "orc_f32_to_f16_array": (None, [P, I64, P]),
        "orc_f16_to_f32_array": (None, [P, I64, P]),
        "orc_quantize_weights_int4_rowwise": (I32, [P, I64, I64, P, P]),
        "orc_quantize_weights_int4_group32": (I32, [P, I64, I64, P, P]),
        "orc_quantize_weights_int8_group32": (I32, [P, I64, I64, P, P]),
        "orc_pack_word": (C.c_uint32, [P]),
        "orc_unpack_word": (None, [C.c_uint32, P]),
        "orc_pack_int4": (I32, [P, I64, I64, P]),
        "orc_unpack_int4": (I32, [P, I64, I64, P]),
        "orc_quantize_act_f32": (I32, [P, I64, I64, P, P]),
        "orc_quantize_act_f16": (I32, [P, I64, I64, P, P]),
        "orc_gemv_w4a8": (I32, [P, P, P, P, F32, I64, I64, P, P]),
        "orc_epilogue_f32": (I32, [P, P, F32, P, I64, P]),
        "orc_gemv_w4a8_group32": (I32, [P, P, P, P, F32, I64, I64, P, P]),
        "orc_gemv_w8a16_group32": (I32, [P, P, P, I64, I64, P]),
        "orc_gemm_w4a8_verify": (I32, [P, P, P, P, P, I64, I64, I64, P, P]),
        "orc_gemv_w4a16": (I32, [P, P, P, P, I64, I64, P]),
        "orc_exp_f32": (C.c_float, [C.c_float]),
        "orc_exp_f32_array": (None, [P, I64, P]),
        "orc_add_rmsnorm_quant": (I32, [P, P, P, F32, I64, I64, P, P, P, P]),
        "orc_swiglu_quant": (I32, [P, I64, I64, P, P, P]),
        "orc_quantize_weights_q6k": (I32, [P, I64, I64, P, P, P]),
        "orc_pack_q6k": (I32, [P, I64, I64, P, P]),
        "orc_unpack_q6k": (I32, [P, P, I64, I64, P]),
        "orc_gemv_q6k_f16": (I32, [P, P, P, P, P, I64, I64, P]),
        "orc_int8x_counts": (None, [P, I64, P, P, P]),
        "orc_int8x_encode": (I32, [P, I64, I64, P, P, P, P, P, P, P]),
        "orc_int8x_decode": (I32, [P, P, P, P, P, P, P, I64, I64, I64, P]),
        "orc_gemv_int8x": (I32, [P, P, P, P, P, P, P, I64, P, F32, F32, I64, I64, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc: int):
    if rc != 0:
        raise OracleError(_ERR.get(rc, f"error {rc}"))


# ---------------------------------------------------------------- fp16 ----
def f32_to_f16(x) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) of fp32 values, RNE."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _lib.orc_f32_to_f16_array(_p(x), x.size, _p(out))
    return out


def f16_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _lib.orc_f16_to_f32_array(_p(h), h.size, _p(out))
    return out


# ------------------------------------------------------ weight quant ----
def quantize_weights_int4_rowwise(W) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row INT4: s_j = max|W_j|/7, q = clip(rne(W/s), -8, 7).  [Orin] derivation."""
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s = np.empty(N, np.float32)
    _check(_lib.orc_quantize_weights_int4_rowwise(_p(W), N, K, _p(q), _p(s)))
    return q, s


def quantize_weights_int4_group32(W) -> Tuple[np.ndarray, np.ndarray]:
    """Q4_0-style: fp16 scale per 32 weights, codes in [-8, 7].  [Ascend] 3.1."""
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s = np.empty((N, K // 32), np.uint16)
    _check(_lib.orc_quantize_weights_int4_group32(_p(W), N, K, _p(q), _p(s)))
    return q, s


def quantize_weights_int8_group32(W) -> Tuple[np.ndarray, np.ndarray]:
    """int8 lm_head: fp16 scale per 32 weights, codes in [-32, 31].  [Ascend] 3.2."""
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s = np.empty((N, K // 32), np.uint16)
    _check(_lib.orc_quantize_weights_int8_group32(_p(W), N, K, _p(q), _p(s)))
    return q, s


# ------------------------------------------------------------ packing ----
def pack_word(q8: Sequence[int]) -> int:
    a = _c(q8, np.int8)
    assert a.size == 8
    return int(_lib.orc_pack_word(_p(a)))


def unpack_word(w: int) -> np.ndarray:
    out = np.empty(8, np.int8)
    _lib.orc_unpack_word(C.c_uint32(w & 0xFFFFFFFF), _p(out))
    return out


def pack_int4(q) -> np.ndarray:
    """[N, K] int8 codes -> [N, K/8] uint32, low nibble first.  [Orin] DP4A section."""
    q = _c(q, np.int8)
    N, K = q.shape
    w = np.empty((N, K // 8), np.uint32)
    _check(_lib.orc_pack_int4(_p(q), N, K, _p(w)))
    return w


def unpack_int4(w, K: Optional[int] = None) -> np.ndarray:
    w = _c(w, np.uint32)
    N, KW = w.shape
    K = KW * 8 if K is None else K
    q = np.empty((N, K), np.int8)
    _check(_lib.orc_unpack_int4(_p(w), N, K, _p(q)))
    return q


# ---------------------------------------------------- activation quant ----
def quantize_act(x) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token INT8: s = max|x|/127, q = clip(rne(x/s), -127, 127).  [Orin] derivation.

    ``x``: float32 or float16 array, [K] or [M, K].  Returns (q int8, s float32)
    with q shaped like x and s of shape [] or [M].
    """
    x = np.asarray(x)
    one = x.ndim == 1
    x2 = x.reshape(1, -1) if one else x
    M, K = x2.shape
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    if x2.dtype == np.float16:
        xb = _c(x2.view(np.uint16), np.uint16)
        _check(_lib.orc_quantize_act_f16(_p(xb), M, K, _p(q), _p(s)))
    else:
        xf = _c(x2, np.float32)
        _check(_lib.orc_quantize_act_f32(_p(xf), M, K, _p(q), _p(s)))
    return (q[0], s[0]) if one else (q, s)


# ------------------------------------------- producers fused with quant ----
def exp_f32(x) -> np.ndarray:
    """e^x in fp32 by Cody-Waite reduction and a degree-7 Taylor polynomial,
    every step one IEEE fp32 operation (the exponential inside SwiGLU)."""
    x = _c(x, np.float32)
    out = np.empty_like(x)
    _lib.orc_exp_f32_array(_p(x), x.size, _p(out))
    return out


def add_rmsnorm_quant(h, delta, gamma, eps: float):
    """Residual add, RMSNorm and per-token quantisation ([Orin] "后续还能继续优化什么",
    items 1-2; textbook RMSNorm).  h, delta fp32 [K] or [M, K] (delta may be
    None), gamma fp32 [K].  Returns (q int8, s fp32, h1 = h + delta, y = the
    normalised fp32 values), shaped like h (s: [] or [M])."""
    h = np.asarray(h)
    one = h.ndim == 1
    h2 = _c(h.reshape(1, -1) if one else h, np.float32)
    M, K = h2.shape
    d = None if delta is None else _c(np.asarray(delta).reshape(M, K), np.float32)
    g = _c(gamma, np.float32)
    if g.size != K:
        raise ValueError("gamma must hold K values")
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    h1 = np.empty((M, K), np.float32)
    y = np.empty((M, K), np.float32)
    _check(_lib.orc_add_rmsnorm_quant(_p(h2), _p(d), _p(g), C.c_float(eps), M, K, _p(h1), _p(y),
                                      _p(q), _p(s)))
    if one:
        return q[0], s[0], h1[0], y[0]
    return q, s, h1, y


def swiglu_quant(gu):
    """SwiGLU h = silu(g) * u of the fused gate/up output gu = [g | u]
    ([M, 2I] or [2I]) and per-token quantisation.  Returns (q int8, s fp32,
    h fp32)."""
    gu = np.asarray(gu)
    one = gu.ndim == 1
    g2 = _c(gu.reshape(1, -1) if one else gu, np.float32)
    M, I2 = g2.shape
    if I2 % 2:
        raise ValueError("gu must hold 2I values per token")
    I = I2 // 2
    q = np.empty((M, I), np.int8)
    s = np.empty(M, np.float32)
    h = np.empty((M, I), np.float32)
    _check(_lib.orc_swiglu_quant(_p(g2), M, I, _p(h), _p(q), _p(s)))
    if one:
        return q[0], s[0], h[0]
    return q, s, h


# ------------------------------------------------- packed 6-bit lm_head ----
def quantize_weights_q6k(W) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q6_K-like weights ([Ascend] 3.2 sizes, this library's own rule): fp32
    W [N, K] (K % 256 == 0) -> (q int8 [N, K] in [-32, 31], sc int8 [N, K/16]
    in [0, 127], d fp16 bits uint16 [N, K/256])."""
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    sc = np.empty((N, K // 16), np.int8)
    d = np.empty((N, K // 256), np.uint16)
    _check(_lib.orc_quantize_weights_q6k(_p(W), N, K, _p(q), _p(sc), _p(d)))
    return q, sc, d


def pack_q6k(q) -> Tuple[np.ndarray, np.ndarray]:
    """int8 codes [N, K] in [-32, 31] -> (ql uint8 [N, K/2], qh uint8 [N, K/4])."""
    q = _c(q, np.int8)
    N, K = q.shape
    ql = np.empty((N, K // 2), np.uint8)
    qh = np.empty((N, K // 4), np.uint8)
    _check(_lib.orc_pack_q6k(_p(q), N, K, _p(ql), _p(qh)))
    return ql, qh


def unpack_q6k(ql, qh) -> np.ndarray:
    ql = _c(ql, np.uint8)
    qh = _c(qh, np.uint8)
    N, K = ql.shape[0], ql.shape[1] * 2
    q = np.empty((N, K), np.int8)
    _check(_lib.orc_unpack_q6k(_p(ql), _p(qh), N, K, _p(q)))
    return q


def gemv_q6k_f16(ql, qh, sc, d, x16) -> np.ndarray:
    """y_j = sum over 16-weight sub-blocks of fp32(d) * sc * sum q x, in binary64."""
    ql = _c(ql, np.uint8)
    qh = _c(qh, np.uint8)
    sc = _c(sc, np.int8)
    d = _c(d, np.uint16)
    xb = _c(x16, np.uint16)
    N, K = ql.shape[0], ql.shape[1] * 2
    y = np.empty(N, np.float64)
    _check(_lib.orc_gemv_q6k_f16(_p(ql), _p(qh), _p(sc), _p(d), _p(xb), N, K, _p(y)))
    return y


# ------------------------------------------------- INT8-X (3,5,8) codec ----
INT8X_BLOCK = 512


def int8x_counts(q) -> Tuple[int, int, int]:
    """Weights of level 1 (|v| <= 3), 2 (|v| <= 15) and 3 (the rest)."""
    q = _c(q, np.int8)
    c = [C.c_int64(), C.c_int64(), C.c_int64()]
    _lib.orc_int8x_counts(_p(q), q.size, *[C.byref(v) for v in c])
    return tuple(int(v.value) for v in c)


def int8x_encode(q, blk: int = INT8X_BLOCK) -> dict:
    """INT8-X (3,5,8) encoding of the row-major flattened int8 tensor q
    ("定長無損 INT8 壓縮與 Triton 融合解碼", sections 2.1-2.5): bitmaps b1, b2,
    streams l1 (3-bit), l2 (5-bit), l3 (bytes), block prefix sums."""
    q = _c(q, np.int8)
    n = q.size
    n1, n2, n3 = int8x_counts(q)
    nb = (n + blk - 1) // blk
    e = dict(b1=np.empty((n + 31) // 32, np.uint32), b2=np.empty(max(1, (n2 + n3 + 31) // 32), np.uint32),
             l1=np.empty(max(1, (3 * n1 + 31) // 32), np.uint32), l2=np.empty(max(1, (5 * n2 + 31) // 32), np.uint32),
             l3=np.empty(max(1, n3), np.uint8), b1_blk=np.empty(nb + 1, np.int32), b2_blk=np.empty(nb + 1, np.int32))
    _check(_lib.orc_int8x_encode(_p(q), n, blk, _p(e["b1"]), _p(e["b2"]), _p(e["l1"]), _p(e["l2"]),
                                 _p(e["l3"]), _p(e["b1_blk"]), _p(e["b2_blk"])))
    e.update(n=n, n1=n1, n2=n2, n3=n3, blk=blk, shape=q.shape)
    return e


def int8x_bits(e: dict) -> int:
    """Payload bits: B1 (n) + B2 (n2 + n3) + 3 n1 + 5 n2 + 8 n3."""
    return e["n"] + e["n2"] + e["n3"] + 3 * e["n1"] + 5 * e["n2"] + 8 * e["n3"]


def int8x_decode(e: dict, t0: int = 0, count: Optional[int] = None) -> np.ndarray:
    count = e["n"] - t0 if count is None else count
    q = np.empty(count, np.int8)
    _check(_lib.orc_int8x_decode(_p(e["b1"]), _p(e["b2"]), _p(e["l1"]), _p(e["l2"]), _p(e["l3"]),
                                 _p(e["b1_blk"]), _p(e["b2_blk"]), e["blk"], t0, count, _p(q)))
    return q


def gemv_int8x(e: dict, qx, sx: float, sw: float) -> Tuple[np.ndarray, np.ndarray]:
    """W8A8 GEMV over INT8-X weights [N, K]: (acc int32 [N], y float64 [N])."""
    N, K = e["shape"]
    qx = _c(qx, np.int8)
    acc = np.empty(N, np.int32)
    y = np.empty(N, np.float64)
    _check(_lib.orc_gemv_int8x(_p(e["b1"]), _p(e["b2"]), _p(e["l1"]), _p(e["l2"]), _p(e["l3"]),
                               _p(e["b1_blk"]), _p(e["b2_blk"]), e["blk"], _p(qx), C.c_float(sx), C.c_float(sw),
                               N, K, _p(acc), _p(y)))
    return acc, y


# -------------------------------------------------------------- GEMVs ----
def gemv_w4a8(w, sw, bias, qx, sx) -> Tuple[np.ndarray, np.ndarray]:
    """acc_j = sum_i qW_ji qx_i (int32), y_j = sW_j sx acc_j + b_j (float64)."""
    w = _c(w, np.uint32)
    N, KW = w.shape
    K = KW * 8
    sw = _c(sw, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    qx = _c(qx, np.int8)
    assert qx.size == K and sw.size == N and (b is None or b.size == N)
    acc = np.empty(N, np.int32)
    y = np.empty(N, np.float64)
    _check(_lib.orc_gemv_w4a8(_p(w), _p(sw), _p(b), _p(qx), C.c_float(float(sx)), N, K,
                              _p(acc), _p(y)))
    return acc, y


def epilogue_f32(sw, bias, sx, acc) -> np.ndarray:
    """y_j in binary32 as the GPU path writes it and a chain hands it on:
    fl32(fl32(sW_j sx) * fl32(acc_j) + b_j) with one rounding (fused)."""
    sw = _c(sw, np.float32)
    acc = _c(acc, np.int32)
    b = None if bias is None else _c(bias, np.float32)
    N = sw.size
    assert acc.size == N and (b is None or b.size == N)
    y = np.empty(N, np.float32)
    _check(_lib.orc_epilogue_f32(_p(sw), _p(b), C.c_float(float(sx)), _p(acc), N, _p(y)))
    return y


def gemv_w4a8_group32(w, s16, bias, qx, sx) -> Tuple[np.ndarray, np.ndarray]:
    """Per-group int32 partials acc_jg and y_j = sx sum_g s_jg acc_jg + b_j."""
    w = _c(w, np.uint32)
    N, KW = w.shape
    K = KW * 8
    s16 = _c(s16, np.uint16)
    b = None if bias is None else _c(bias, np.float32)
    qx = _c(qx, np.int8)
    assert qx.size == K and s16.shape == (N, K // 32)
    accg = np.empty((N, K // 32), np.int32)
    y = np.empty(N, np.float64)
    _check(_lib.orc_gemv_w4a8_group32(_p(w), _p(s16), _p(b), _p(qx), C.c_float(float(sx)),
                                      N, K, _p(accg), _p(y)))
    return accg, y


def gemv_w8a16_group32(w8, s16, x16) -> np.ndarray:
    """y_j = sum_g s_jg sum_{i in g} q_ji x_i with fp16 x (uint16 bit patterns or float16)."""
    w8 = _c(w8, np.int8)
    N, K = w8.shape
    s16 = _c(s16, np.uint16)
    x16 = np.asarray(x16)
    xb = _c(x16.view(np.uint16) if x16.dtype == np.float16 else x16, np.uint16)
    assert xb.size == K and s16.shape == (N, K // 32)
    y = np.empty(N, np.float64)
    _check(_lib.orc_gemv_w8a16_group32(_p(w8), _p(s16), _p(xb), N, K, _p(y)))
    return y


def gemv_w4a16(w, sw, bias, x16) -> np.ndarray:
    """W4A16 comparison GEMV: packed per-row INT4 weights against fp16 x
    (uint16 bit patterns), y = sW * sum q x + b in binary64."""
    w = _c(w, np.uint32)
    N = w.shape[0]
    K = w.shape[1] * 8
    sw = _c(sw, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    xb = _c(x16, np.uint16)
    y = np.empty(N, np.float64)
    _check(_lib.orc_gemv_w4a16(_p(w), _p(sw), _p(b), _p(xb), N, K, _p(y)))
    return y


def gemm_w4a8_verify(w, sw, bias, qx, sx) -> Tuple[np.ndarray, np.ndarray]:
    """M tokens at once: qx [M, K], sx [M] -> acc [M, N] int32, y [M, N] float64."""
    w = _c(w, np.uint32)
    N, KW = w.shape
    K = KW * 8
    sw = _c(sw, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    qx = _c(qx, np.int8)
    M = qx.shape[0]
    sx = _c(sx, np.float32)
    assert qx.shape == (M, K) and sx.size == M
    acc = np.empty((M, N), np.int32)
    y = np.empty((M, N), np.float64)
    _check(_lib.orc_gemm_w4a8_verify(_p(w), _p(sw), _p(b), _p(qx), _p(sx), M, N, K,
                                     _p(acc), _p(y)))
    return acc, y


# ------------------------------------------------------- compositions ----
def prepare_int4_rowwise(W):
    """Load-time preparation of one linear: quantise per row, then pack."""
    q, s = quantize_weights_int4_rowwise(W)
    return pack_int4(q), s


def prepare_int4_group32(W):
    q, s16 = quantize_weights_int4_group32(W)
    return pack_int4(q), s16


def linear_w4a8(w, sw, bias, x) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """One decode linear: quantise the activation, then the W4A8 GEMV.
    Returns (qx, sx, acc, y)."""
    qx, sx = quantize_act(x)
    acc, y = gemv_w4a8(w, sw, bias, qx, sx)
    return qx, sx, acc, y


def chain_w4a8(linears, x0):
    """A decoder's chain of per-row W4A8 linears ([Orin] derivation section,
    one linear after another): linear t quantises its activation, takes the
    GEMV, and linear t+1's activation is the first K_{t+1} values of linear
    t's binary32 output (epilogue_f32).  linears: (w, sw, bias) with w the
    packed [N, K/8] words.  Returns per linear (qx, sx, acc, y64, y32)."""
    out, x = [], np.asarray(x0, np.float32)
    for t, (w, sw, b) in enumerate(linears):
        K = np.asarray(w).shape[1] * 8
        assert x.size == K, (t, x.size, K)
        qx, sx, acc, y64 = linear_w4a8(w, sw, b, x)
        y32 = epilogue_f32(sw, b, sx, acc)
        out.append((qx, sx, acc, y64, y32))
        if t + 1 < len(linears):
            x = y32[:np.asarray(linears[t + 1][0]).shape[1] * 8]
    return out


def linear_w4a8_group32(w, s16, bias, x):
    qx, sx = quantize_act(x)
    accg, y = gemv_w4a8_group32(w, s16, bias, qx, sx)
    return qx, sx, accg, y


def rel_err_plain(y_test, y_ref, floor: float = 1e-3) -> float:
    """max |y_test - y_ref| / |y_ref| over the rows with |y_ref| >= floor *
    max |y_ref| (0 when there is none): the plain relative error reported
    beside the gated one of ``rel_err_rowwise``."""
    yt = np.asarray(y_test, np.float64).ravel()
    yr = np.asarray(y_ref, np.float64).ravel()
    if yr.size == 0:
        return 0.0
    big = np.abs(yr) >= floor * np.abs(yr).max()
    big &= np.abs(yr) > 0
    if not big.any():
        return 0.0
    return float((np.abs(yt[big] - yr[big]) / np.abs(yr[big])).max())


def rel_err_rowwise(y_test, y_ref, sw, sx, acc, bias) -> np.ndarray:
    """|y_test - y_ref| / m_j with m_j = |sW_j sx acc_j| + |b_j|: the error
    relative to the row's magnitude before cancellation (0/0 counts as 0)."""
    m = np.abs(np.asarray(sw, np.float64) * np.float64(sx) * np.asarray(acc, np.float64))
    if bias is not None:
        m = m + np.abs(np.asarray(bias, np.float64))
    d = np.abs(np.asarray(y_test, np.float64) - np.asarray(y_ref, np.float64))
    return np.where(m > 0, d / np.where(m > 0, m, 1.0), np.where(d > 0, np.inf, 0.0))
