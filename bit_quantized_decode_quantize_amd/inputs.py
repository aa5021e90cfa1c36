"""Seeded synthetic inputs for the W4A8 decode GEMV path.

This module is the only code that both the GPU path's tests/bench and the
CPU oracle consume.  It holds none of the method's arithmetic: no
quantisation, no packing, no dot products, no scales.  It only draws
numbers and shapes them into the value distributions of the workloads the
pages measure (fp32 weights ~N(0, 0.02^2), activations ~N(0, 1), biases
~N(0, 0.01^2), SwiGLU-shaped activations for the down projection).

Generator: counter-based SplitMix64 (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014; the 64-bit finaliser with
Vigna's published constants).  Draw ``i`` of a stream is the SplitMix64
output for state ``key + (i + 1) * GOLDEN``, so any element can be computed
on its own, in any order, on any device.  Uniforms take the top 53 bits;
normals use the Box-Muller transform (one cosine branch per pair of draws).

The integer part is bit-identical on every device.  Box-Muller evaluates
log/sqrt/cos in float64; CPU and GPU maths libraries may differ in the last
float64 bit, which can (rarely) move an fp32 result by one ulp.  Every test
therefore hands the *same buffer* to the oracle and to the GPU path.

Everything here is plain torch, so it runs on the CPU or, for multi-GB
weight streams, on the GPU (``device="cuda"``).
"""
from __future__ import annotations

import math
from typing import Dict, Iterator, Tuple

import torch

_M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
_C1 = 0xBF58476D1CE4E5B9
_C2 = 0x94D049BB133111EB


def _s64(v: int) -> int:
    """Python int in [0, 2^64) -> the int64 with the same bit pattern."""
    v &= _M64
    return v - (1 << 64) if v >= (1 << 63) else v


def _mix64_int(z: int) -> int:
    """SplitMix64 finaliser on a Python int (exact, for key derivation)."""
    z &= _M64
    z = ((z ^ (z >> 30)) * _C1) & _M64
    z = ((z ^ (z >> 27)) * _C2) & _M64
    return z ^ (z >> 31)


def _fnv1a64(s: str) -> int:
    h = 0xCBF29CE484222325
    for b in s.encode("utf-8"):
        h ^= b
        h = (h * 0x100000001B3) & _M64
    return h


def stream_key(seed: int, name: str) -> int:
    """64-bit key of the named stream (tensor) under ``seed``."""
    return _mix64_int(_mix64_int((seed + GOLDEN) & _M64) ^ _fnv1a64(name))


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return torch.bitwise_right_shift(z, k) & ((1 << (64 - k)) - 1)


def _mix64(z: torch.Tensor) -> torch.Tensor:
    # int64 multiplication wraps modulo 2^64 on every torch backend.
    z = (z ^ _lsr(z, 30)) * _s64(_C1)
    z = (z ^ _lsr(z, 27)) * _s64(_C2)
    return z ^ _lsr(z, 31)


def raw_u64(key: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Draws ``start .. start+count-1`` of stream ``key`` as int64 bit patterns."""
    idx = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    state = idx * _s64(GOLDEN) + _s64(key)
    return _mix64(state)


def _uniform53(z: torch.Tensor) -> torch.Tensor:
    """(top 53 bits + 0.5) * 2^-53: float64 in the open interval (0, 1)."""
    return (_lsr(z, 11).to(torch.float64) + 0.5) * (2.0 ** -53)


_CHUNK = 1 << 26


def _normal_f64(key: int, start: int, count: int, device) -> torch.Tensor:
    z = raw_u64(key, 2 * start, 2 * count, device).view(count, 2)
    u1 = _uniform53(z[:, 0])
    u2 = _uniform53(z[:, 1])
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def normal(name: str, shape, sigma: float = 1.0, seed: int = 0, device="cpu",
           dtype=torch.float32) -> torch.Tensor:
    """N(0, sigma^2) values, computed in float64 and rounded once to fp32.

    ``dtype=torch.float16`` rounds the fp32 value to fp16 (RNE).
    """
    shape = tuple(int(s) for s in (shape if isinstance(shape, (tuple, list)) else (shape,)))
    n = 1
    for s in shape:
        n *= s
    key = stream_key(seed, name)
    out = torch.empty(n, dtype=torch.float32, device=device)
    for a in range(0, n, _CHUNK):
        c = min(_CHUNK, n - a)
        out[a:a + c] = (_normal_f64(key, a, c, device) * sigma).to(torch.float32)
    out = out.view(shape)
    if dtype == torch.float16:
        out = out.to(torch.float16)
    elif dtype != torch.float32:
        raise ValueError("dtype must be float32 or float16")
    return out


def uniform_int(name: str, shape, lo: int, hi: int, seed: int = 0, device="cpu",
                dtype=torch.int32) -> torch.Tensor:
    """Integers uniform on [lo, hi] (multiply-shift on the top 32 bits)."""
    shape = tuple(int(s) for s in (shape if isinstance(shape, (tuple, list)) else (shape,)))
    n = 1
    for s in shape:
        n *= s
    span = hi - lo + 1
    assert 0 < span <= (1 << 31)
    z = raw_u64(stream_key(seed, name), 0, n, device)
    top = _lsr(z, 32)                       # [0, 2^32)
    v = _lsr(top * span, 32) + lo           # top*span < 2^63: no overflow
    return v.to(dtype).view(shape)


def int8_codes_by_band(name: str, shape, shares=(555, 404, 41), seed: int = 0, device="cpu") -> torch.Tensor:
    """int8 weight codes whose magnitude falls in the bands 0..3, 4..15 and
    16..127 with probabilities shares / 1000 (default: the shares the INT8-X
    page reports for its model), uniform within a band, random sign."""
    band = uniform_int(f"{name}/band", shape, 0, 999, seed, device)
    m1 = uniform_int(f"{name}/m1", shape, 0, 3, seed, device)
    m2 = uniform_int(f"{name}/m2", shape, 4, 15, seed, device)
    m3 = uniform_int(f"{name}/m3", shape, 16, 127, seed, device)
    neg = uniform_int(f"{name}/sign", shape, 0, 1, seed, device)
    mag = torch.where(band < shares[0], m1, torch.where(band < shares[0] + shares[1], m2, m3))
    return torch.where(neg == 1, -mag, mag).to(torch.int8)


def random_words(name: str, shape, seed: int = 0, device="cpu") -> torch.Tensor:
    """Uniformly random 32-bit words (every nibble pattern), as int32."""
    shape = tuple(int(s) for s in (shape if isinstance(shape, (tuple, list)) else (shape,)))
    n = 1
    for s in shape:
        n *= s
    z = raw_u64(stream_key(seed, name), 0, n, device)
    lo32 = z & 0xFFFFFFFF
    lo32 = torch.where(lo32 >= (1 << 31), lo32 - (1 << 32), lo32)
    return lo32.to(torch.int32).view(shape)


def distinct_indices(name: str, n: int, count: int, seed: int = 0) -> torch.Tensor:
    """``count`` distinct indices in [0, n): the ``count`` smallest random keys."""
    keys = raw_u64(stream_key(seed, name), 0, n, "cpu")
    keys = _lsr(keys, 1)                    # non-negative, order-preserving on the top 63 bits
    order = torch.argsort(keys, stable=True)
    return torch.sort(order[:count]).values


def with_outliers(x: torch.Tensor, name: str, frac: float = 0.01, factor: float = 20.0,
                  seed: int = 0) -> torch.Tensor:
    """Multiply round(frac * K) distinct entries of the 1-D ``x`` by ``factor``."""
    k = x.numel()
    m = int(round(frac * k))
    idx = distinct_indices(name, k, m, seed).to(x.device)
    y = x.clone()
    y[idx] = y[idx] * factor
    return y


def swiglu_like(name: str, K: int, seed: int = 0, device="cpu",
                dtype=torch.float32) -> torch.Tensor:
    """silu(g) * u with g, u ~ N(0, 1): the shape of a down-projection input."""
    g = normal(name + "/g", K, 1.0, seed, device).to(torch.float64)
    u = normal(name + "/u", K, 1.0, seed, device).to(torch.float64)
    v = (g / (1.0 + torch.exp(-g)) * u).to(torch.float32)
    return v.to(torch.float16) if dtype == torch.float16 else v


# --------------------------------------------------------------------------
# Workload shapes (Qwen2-7B-shaped decoder, Gemma-shaped group-32 decoder)
# --------------------------------------------------------------------------

QWEN = dict(hidden=3584, kv_dim=512, inter=18944, layers=28, vocab=152064)
GEMMA = dict(hidden=1536, qkv_rows=2048, o_in=2048, ffn=6144, layers=35, vocab=262144)


def qwen_layer_linears() -> Tuple[Tuple[str, int, int], ...]:
    """(name, N rows, K) of the four GEMVs of one decoder layer after fusion:
    QKV = Q(3584) + K(512) + V(512) rows; gate/up = 2 x 18944 rows."""
    h, kv, i = QWEN["hidden"], QWEN["kv_dim"], QWEN["inter"]
    return (("qkv", h + 2 * kv, h), ("o", h, h), ("gate_up", 2 * i, h), ("down", h, i))


def gemma_layer_linears() -> Tuple[Tuple[str, int, int], ...]:
    g = GEMMA
    return (("qkv", g["qkv_rows"], g["hidden"]), ("o", g["hidden"], g["o_in"]),
            ("gate_up", 2 * g["ffn"], g["hidden"]), ("down", g["hidden"], g["ffn"]))


def linear_input(prefix: str, name: str, K: int, seed: int, device, dtype=torch.float32):
    """Activation feeding one linear: N(0,1), or silu(g)*u for the down projection."""
    if name == "down":
        return swiglu_like(f"{prefix}/{name}/x", K, seed, device, dtype)
    return normal(f"{prefix}/{name}/x", K, 1.0, seed, device, dtype)


def single_gemv_inputs(seed: int = 0, device="cpu", K: int = 3584, N: int = 3584) -> Dict[str, torch.Tensor]:
    """One Q-projection GEMV: W ~N(0, 0.02^2) [N, K], x ~N(0, 1) with 1% of
    entries x20, bias ~N(0, 0.01^2)."""
    W = normal("single/W", (N, K), 0.02, seed, device)
    x = with_outliers(normal("single/x", K, 1.0, seed, device), "single/outliers", seed=seed)
    b = normal("single/b", N, 0.01, seed, device)
    return dict(W=W, x=x, b=b)
