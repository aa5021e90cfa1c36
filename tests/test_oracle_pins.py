"""Pins of the CPU oracle against facts other than itself.

Each test checks the oracle against a value the pages print, a closed form,
an invariant, a library routine (numpy's IEEE float16, Python's round-half-
even ``round``, numpy's integer and float64 matmul) or brute force on tiny
inputs.  None of them re-types the oracle's own formula as the expected
value.  Pages cited:
  [Orin]   "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到 24 tok/s"
  [Ascend] "在香橙派上跑 Gemma4：vLLM 适配昇腾 310B 的内核开发实录"
"""
import os
import subprocess

import numpy as np
import pytest

import oracle as O
from bit_quantized_decode_quantize_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ints(s):
    return [int(v, 0) for v in s.split()]


def _floats(s):
    return [float(v) for v in s.split()]


# ------------------------------------------------------------------ fp16 --
def test_f16_to_f32_exhaustive_vs_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    got = O.f16_to_f32(h)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f32_patterns():
    rng = np.random.default_rng(1234)
    parts = []
    # every (sign, exponent, top-10 mantissa bits) with low-13-bit endings at and
    # around the rounding tie of the normal fp16 range
    hi = np.arange(1 << 19, dtype=np.uint64) << np.uint64(13)
    for low in (0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF):
        parts.append((hi | np.uint64(low)).astype(np.uint32))
    # the fp16 subnormal / underflow range (fp32 exponents 100..113), random
    e = rng.integers(100, 114, size=2_000_000, dtype=np.uint32)
    m = rng.integers(0, 1 << 23, size=e.size, dtype=np.uint32)
    s = rng.integers(0, 2, size=e.size, dtype=np.uint32)
    parts.append((s << 31) | (e << 23) | m)
    # exact ties in the subnormal range: odd multiples of 2^-25 (half a quantum)
    k = np.arange(0, 2048, dtype=np.float64)
    parts.append(((2 * k + 1) * 2.0 ** -25).astype(np.float32).view(np.uint32))
    # overflow boundary and random patterns everywhere
    parts.append(np.array([0x477FE000, 0x477FEFFF, 0x477FF000, 0x477FF001, 0x7F7FFFFF,
                           0x7F800000, 0xFF800000, 0x00000001, 0x80000000], np.uint32))
    parts.append(rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32))
    return np.concatenate(parts).view(np.float32)


def test_f32_to_f16_rne_vs_numpy():
    x = _f32_patterns()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = O.f32_to_f16(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


# ------------------------------------------------------------- packing --
def test_word_layout_golden(golden):
    g = golden("int4_word_layout.txt")
    assert O.pack_word(_ints(g["codes"])) == int(g["word"], 16)
    assert list(O.unpack_word(int(g["word"], 16))) == _ints(g["codes"])
    assert O.pack_word([-1, 0, 0, 0, 0, 0, 0, 0]) == int(g["single_w0_minus1"], 16)
    assert O.pack_word([0, 0, 0, 0, 0, 0, 0, -8]) == int(g["single_w7_minus8"], 16)


def test_every_code_at_every_position():
    for k in range(8):
        for v in range(-8, 8):
            q = [0] * 8
            q[k] = v
            w = O.pack_word(q)
            assert w == ((v & 0xF) << (4 * k))          # nibble k holds v mod 16
            assert list(O.unpack_word(w)) == q


def test_pack_unpack_roundtrip_exhaustive(tmp_path):
    """pack(unpack(w)) == w over all 2^32 words (OpenMP helper in C)."""
    exe = tmp_path / "prt"
    odir = os.path.join(ROOT, "oracle")
    subprocess.run(["gcc", "-O2", "-fopenmp", os.path.join(ROOT, "tests/helpers/pack_roundtrip.c"),
                    "-o", str(exe), f"-L{odir}", "-loracle", f"-Wl,-rpath,{odir}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches=0 out_of_range=0" in r.stdout


def test_matrix_pack_is_wordwise_and_rejects_out_of_range():
    q = I.uniform_int("pin/packq", (5, 48), -8, 7).numpy().astype(np.int8)
    w = O.pack_int4(q)
    assert w.shape == (5, 6)
    for j in range(5):
        for t in range(6):
            assert w[j, t] == O.pack_word(q[j, 8 * t:8 * t + 8])
    assert np.array_equal(O.unpack_int4(w), q)
    bad = q.copy()
    bad[2, 3] = 8
    with pytest.raises(O.OracleError):
        O.pack_int4(bad)
    with pytest.raises(O.OracleError):
        O.pack_int4(np.zeros((2, 12), np.int8))


def test_row_bytes_golden(golden):
    g = golden("row_bytes.txt")
    K = int(g["hidden"])
    w = O.pack_int4(np.zeros((3, K), np.int8))
    assert w.nbytes // 3 == int(g["int4_bytes"])
    assert K * 1 == int(g["int8_bytes"]) and K * 2 == int(g["fp16_bytes"])


# --------------------------------------------------- activation quant --
def test_act_quant_rne_golden(golden):
    g = golden("act_quant_rne.txt")
    x = np.array(_floats(g["x"]), np.float32)
    q, s = O.quantize_act(x)
    assert float(s) == float(g["s"])
    assert list(q) == _ints(g["q"])
    assert list(q) != _ints(g["q_half_away"])


def _act_ref_python(x):
    """Independent route: numpy fp32 division + Python's round-half-even."""
    x = np.asarray(x, np.float32)
    amax = np.float32(np.max(np.abs(x)))
    s = np.float32(amax / np.float32(127.0))
    if s == 0:
        return [0] * x.size, s
    q = [max(-127, min(127, round(float(np.float32(v / s))))) for v in x]
    return q, s


def test_act_quant_brute_force_vs_python_round():
    for t in range(40):
        K = 8 + 8 * (t % 9)
        x = I.normal(f"pin/act/{t}", K, 10.0 ** ((t % 7) - 3)).numpy()
        if t % 5 == 0:   # many exact ties: half-integers scaled so that s = 1
            x = (np.round(x * 4) / 2).astype(np.float32)
            x[0] = 127.0
        q, s = O.quantize_act(x)
        qr, sr = _act_ref_python(x)
        assert s.view(np.uint32) == sr.view(np.uint32)
        assert list(q) == qr


def test_act_quant_invariants():
    x = I.with_outliers(I.normal("pin/act/inv", 3584), "pin/act/inv/o").numpy()
    q, s = O.quantize_act(x)
    assert np.abs(q.astype(int)).max() == 127 and q.min() >= -127
    i = int(np.argmax(np.abs(x)))
    assert q[i] == (127 if x[i] > 0 else -127)
    for k in (-20, -3, 5, 30):          # power-of-two scaling is exact in fp32
        q2, s2 = O.quantize_act(np.ldexp(x, k).astype(np.float32))
        assert np.array_equal(q2, q) and s2 == np.float32(np.ldexp(s, k))
    qn, sn = O.quantize_act(-x)
    assert np.array_equal(qn, -q) and sn == s
    qz, sz = O.quantize_act(np.zeros(64, np.float32))
    assert sz == 0 and not qz.any()
    with pytest.raises(O.OracleError):
        O.quantize_act(np.array([1.0, np.nan] + [0.0] * 6, np.float32))
    with pytest.raises(O.OracleError):
        O.quantize_act(np.array([1.0, np.inf] + [0.0] * 6, np.float32))


def test_act_quant_fp16_equals_widened_fp32():
    x16 = I.normal("pin/act/f16", (3, 1536), 1.0, dtype=__import__("torch").float16).numpy()
    q16, s16 = O.quantize_act(x16)
    q32, s32 = O.quantize_act(x16.astype(np.float32))
    assert np.array_equal(q16, q32) and np.array_equal(s16, s32)


# ------------------------------------------------------- weight quant --
def _round_div(W, s):
    """clip(round(W/s)) via numpy fp32 division and Python round()."""
    out = np.zeros(W.shape, np.int64)
    for idx in np.ndindex(W.shape):
        if s[idx[:-1]] != 0:
            out[idx] = round(float(np.float32(W[idx] / s[idx[:-1]])))
    return out


def test_weight_quant_rowwise_vs_python():
    W = I.normal("pin/wq", (7, 64), 0.02).numpy()
    W[3] = 0.0                                       # all-zero row
    W[5, 10] = -0.5                                  # a dominant negative entry
    q, s = O.quantize_weights_int4_rowwise(W)
    amax = np.max(np.abs(W), axis=1)
    assert np.array_equal(s, (amax / np.float32(7.0)).astype(np.float32))
    ref = np.clip(_round_div(W, s), -8, 7)
    assert np.array_equal(q.astype(np.int64), ref)
    assert not q[3].any() and s[3] == 0
    assert q[5, 10] == -7
    # quantisation error bound |W - s q| <= s/2 (nothing clips under max/7)
    err = np.abs(W.astype(np.float64) - s[:, None].astype(np.float64) * q)
    assert np.all(err <= s[:, None].astype(np.float64) / 2 * (1 + 1e-6))
    assert np.all(np.abs(q[s > 0]).max(axis=1) == 7)


def test_weight_quant_group32_vs_numpy_fp16():
    W = I.normal("pin/wq32", (5, 96), 0.02).numpy()
    W[1, 32:64] = 0.0                                # an all-zero group
    q, s16 = O.quantize_weights_int4_group32(W)
    amax = np.max(np.abs(W.reshape(5, 3, 32)), axis=2)
    ref_s16 = (amax / np.float32(7.0)).astype(np.float32).astype(np.float16)
    assert np.array_equal(s16, ref_s16.view(np.uint16))
    sg = ref_s16.astype(np.float32)
    ref = np.clip(_round_div(W.reshape(5, 3, 32), sg), -8, 7).reshape(5, 96)
    assert np.array_equal(q.astype(np.int64), ref)
    assert not q[1, 32:64].any()


def test_weight_quant_int8_group32_vs_numpy_fp16():
    W = I.normal("pin/wq8", (4, 64), 0.02).numpy()
    q, s16 = O.quantize_weights_int8_group32(W)
    amax = np.max(np.abs(W.reshape(4, 2, 32)), axis=2)
    ref_s16 = (amax / np.float32(31.0)).astype(np.float32).astype(np.float16)
    assert np.array_equal(s16, ref_s16.view(np.uint16))
    ref = np.clip(_round_div(W.reshape(4, 2, 32), ref_s16.astype(np.float32)), -32, 31)
    assert np.array_equal(q.astype(np.int64), ref.reshape(4, 64))
    assert q.min() >= -32 and q.max() <= 31


# ------------------------------------------------------------- GEMVs --
def test_int32_bound_golden(golden):
    g = golden("int32_bound.txt")
    K = int(g["hidden"])
    assert int(g["max_abs_qw"]) * int(g["max_abs_qx"]) == int(g["max_term"])
    w = O.pack_int4(np.full((2, K), -8, np.int8))
    sw = np.ones(2, np.float32)
    acc, _ = O.gemv_w4a8(w, sw, None, np.full(K, -127, np.int8), 1.0)
    assert list(acc) == [int(g["row_bound"])] * 2
    acc, _ = O.gemv_w4a8(w, sw, None, np.full(K, 127, np.int8), 1.0)
    assert list(acc) == [-int(g["row_bound"])] * 2
    assert int(g["row_bound"]) < int(g["int32_max"]) == 2 ** 31 - 1
    # the down projection's reduction length, same argument: 18944 * 1016
    K2 = 18944
    w2 = O.pack_int4(np.full((1, K2), -8, np.int8))
    acc2, _ = O.gemv_w4a8(w2, np.ones(1, np.float32), None, np.full(K2, -127, np.int8), 1.0)
    assert acc2[0] == K2 * int(g["max_term"]) == 19247104


@pytest.mark.parametrize("N,K", [(1, 8), (3, 16), (9, 32), (4, 40), (7, 64), (2, 3584)])
def test_gemv_acc_brute_force_vs_numpy_matmul(N, K):
    q = I.uniform_int(f"pin/gq/{N}/{K}", (N, K), -8, 7).numpy().astype(np.int8)
    q[0, 0] = -8
    qx = I.uniform_int(f"pin/gx/{N}/{K}", K, -127, 127).numpy().astype(np.int8)
    w = O.pack_int4(q)
    sw = I.normal(f"pin/gs/{N}/{K}", N, 0.01).numpy()
    b = I.normal(f"pin/gb/{N}/{K}", N, 0.01).numpy()
    acc, y = O.gemv_w4a8(w, sw, b, qx, np.float32(0.37))
    ref = q.astype(np.int64) @ qx.astype(np.int64)
    assert np.array_equal(acc.astype(np.int64), ref)
    # the same integer through DP4A's pairing: dot4(w0..3, x0..3) + dot4(w4..7, x4..7)
    lo = q.reshape(N, -1, 8)[:, :, :4].astype(np.int64)
    hi = q.reshape(N, -1, 8)[:, :, 4:].astype(np.int64)
    xl = qx.reshape(-1, 8)[:, :4].astype(np.int64)
    xh = qx.reshape(-1, 8)[:, 4:].astype(np.int64)
    assert np.array_equal(acc.astype(np.int64), (lo * xl).sum((1, 2)) + (hi * xh).sum((1, 2)))
    # bias off: y scales with acc alone
    _, y0 = O.gemv_w4a8(w, sw, None, qx, np.float32(0.37))
    assert np.allclose(y - y0, b.astype(np.float64), rtol=0, atol=1e-15)


def test_gemv_closed_form_bound_against_unquantised_math():
    """|y - (Wx + b)| <= sum_i (s_j/2 |x_i| + |W_ji| s^x/2 + s_j s^x/4):
    |W - s q| <= s/2 and |x - s^x q^x| <= s^x/2 ([Orin] derivation)."""
    d = I.single_gemv_inputs(seed=3, N=256, K=3584)
    W, x, b = d["W"].numpy(), d["x"].numpy(), d["b"].numpy()
    w, s = O.prepare_int4_rowwise(W)
    qx, sx, acc, y = O.linear_w4a8(w, s, b, x)
    exact = W.astype(np.float64) @ x.astype(np.float64) + b
    s64, sx64 = s.astype(np.float64), float(sx)
    bound = (s64 / 2)[:, None] * np.abs(x)[None, :] + np.abs(W) * sx64 / 2 + (s64[:, None] * sx64 / 4)
    bound = bound.sum(1) * (1 + 1e-9) + 1e-12
    assert np.all(np.abs(y - exact) <= bound)
    # and the quantised result is a real approximation, not a trivially loose one
    assert np.median(np.abs(y - exact) / (np.abs(exact) + 1e-3)) < 0.2


def test_gemv_invariants_permutation_and_linearity():
    q = I.uniform_int("pin/inv/q", (16, 64), -8, 7).numpy().astype(np.int8)
    w = O.pack_int4(q)
    sw = np.ones(16, np.float32)
    x1 = I.uniform_int("pin/inv/x1", 64, -60, 60).numpy().astype(np.int8)
    x2 = I.uniform_int("pin/inv/x2", 64, -60, 60).numpy().astype(np.int8)
    a1, _ = O.gemv_w4a8(w, sw, None, x1, 1.0)
    a2, _ = O.gemv_w4a8(w, sw, None, x2, 1.0)
    a12, _ = O.gemv_w4a8(w, sw, None, (x1 + x2).astype(np.int8), 1.0)
    assert np.array_equal(a12, a1 + a2)
    perm = I.distinct_indices("pin/inv/perm", 16, 16).numpy()
    ap, _ = O.gemv_w4a8(w[perm], sw, None, x1, 1.0)
    assert np.array_equal(ap, a1[perm])


def test_fused_rows_equal_separate_gemvs(golden):
    """[Ascend] 3.1: concatenated q/k/v (and gate/up) rows stay a valid weight,
    so one GEMV over the fused rows equals the separate GEMVs bit for bit."""
    K = 256
    parts = [I.normal(f"pin/fuse/{n}", (r, K), 0.02).numpy() for n, r in (("q", 24), ("k", 8), ("v", 8))]
    bs = [I.normal(f"pin/fuse/b/{i}", p.shape[0], 0.01).numpy() for i, p in enumerate(parts)]
    x = I.normal("pin/fuse/x", K).numpy()
    sep = [O.linear_w4a8(*O.prepare_int4_rowwise(p), b, x) for p, b in zip(parts, bs)]
    wf, sf = O.prepare_int4_rowwise(np.concatenate(parts))
    _, _, accf, yf = O.linear_w4a8(wf, sf, np.concatenate(bs), x)
    assert np.array_equal(accf, np.concatenate([r[2] for r in sep]))
    assert np.array_equal(yf, np.concatenate([r[3] for r in sep]))
    g = golden("fused_launches.txt")
    assert int(g["layers"]) * 7 == int(g["launches_unfused"])
    assert int(g["layers"]) * 4 == int(g["launches_fused"])


def test_gemv_group32_equal_scales_reduce_to_rowwise():
    """With every 32-group at the same max |W| = 7 * 2^-6, every fp16 group
    scale and the fp32 row scale are exactly 2^-6: the group partials sum to
    the per-row accumulator and both outputs agree."""
    N, K = 6, 128
    W = I.normal("pin/g32eq", (N, K), 0.02).numpy()
    W = np.clip(W, -0.1, 0.1)
    W[:, ::32] = np.float32(7 * 2.0 ** -6) * np.where(np.arange(N)[:, None] % 2, 1, -1)
    b = I.normal("pin/g32eq/b", N, 0.01).numpy()
    x = I.normal("pin/g32eq/x", K).numpy()
    wr, sr = O.prepare_int4_rowwise(W)
    wg, sg = O.prepare_int4_group32(W)
    assert np.all(sr == np.float32(2.0 ** -6)) and np.all(O.f16_to_f32(sg) == np.float32(2.0 ** -6))
    assert np.array_equal(wr, wg)
    _, _, acc, yr = O.linear_w4a8(wr, sr, b, x)
    _, _, accg, yg = O.linear_w4a8_group32(wg, sg, b, x)
    assert np.array_equal(accg.sum(1), acc)
    assert np.array_equal(yr, yg)


def test_gemv_group32_vs_numpy_float64():
    N, K = 9, 192
    q = I.uniform_int("pin/g32/q", (N, K), -8, 7).numpy().astype(np.int8)
    s16 = O.f32_to_f16(np.abs(I.normal("pin/g32/s", (N, K // 32), 0.003).numpy()) + 1e-4)
    qx = I.uniform_int("pin/g32/x", K, -127, 127).numpy().astype(np.int8)
    b = I.normal("pin/g32/b", N, 0.01).numpy()
    sx = np.float32(0.0421)
    accg, y = O.gemv_w4a8_group32(O.pack_int4(q), s16, b, qx, sx)
    ref_g = np.einsum("ngk,gk->ng", q.reshape(N, -1, 32).astype(np.int64), qx.reshape(-1, 32).astype(np.int64))
    assert np.array_equal(accg.astype(np.int64), ref_g)
    sg = s16.view(np.float16).astype(np.float64)
    ref = float(sx) * (sg * ref_g).sum(1) + b
    assert np.allclose(y, ref, rtol=1e-14, atol=0)


def test_gemv_w8a16_vs_numpy_float64_dequantised_matmul():
    N, K = 11, 160
    W = I.normal("pin/w8", (N, K), 0.02).numpy()
    q, s16 = O.quantize_weights_int8_group32(W)
    q[2, 5] = -32                                     # the code range's negative end
    x16 = I.normal("pin/w8/x", K, 1.0, dtype=__import__("torch").float16).numpy()
    y = O.gemv_w8a16_group32(q, s16, x16)
    deq = q.astype(np.float64) * np.repeat(s16.view(np.float16).astype(np.float64), 32, axis=1)
    ref = deq @ x16.astype(np.float64)
    mag = np.abs(deq) @ np.abs(x16.astype(np.float64))
    assert np.all(np.abs(y - ref) <= 1e-13 * mag + 1e-300)


def _np_unpack_codes(w):
    """Signed INT4 codes of packed words with numpy bit operations (nibble k
    of a word is code k, two's complement)."""
    w = np.asarray(w, np.uint32)
    nib = (w[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF
    q = nib.astype(np.int64)
    q = np.where(q >= 8, q - 16, q)
    return q.reshape(*w.shape[:-1], w.shape[-1] * 8)


def test_gemv_w4a16_vs_numpy_float64():
    """The float-unpack comparison GEMV: codes unpacked by numpy, a float64
    matmul against the fp16 x; every product and (for these sizes) every
    partial sum is exact in binary64, so only the final rounding differs."""
    N, K = 13, 256
    W = I.normal("pin/w4a16/W", (N, K), 0.02).numpy()
    w, s = O.prepare_int4_rowwise(W)
    w[3, 0] = 0x88888888                               # eight -8 codes
    b = I.normal("pin/w4a16/b", N, 0.01).numpy()
    x16 = I.normal("pin/w4a16/x", K, 1.0, dtype=__import__("torch").float16).numpy()
    y = O.gemv_w4a16(w, s, b, x16.view(np.uint16))
    q = _np_unpack_codes(w)
    assert q[3, :8].tolist() == [-8] * 8
    ref = s.astype(np.float64) * (q.astype(np.float64) @ x16.astype(np.float64)) + b.astype(np.float64)
    mag = np.abs(s.astype(np.float64)) * (np.abs(q) @ np.abs(x16.astype(np.float64))) + np.abs(b)
    assert np.all(np.abs(y - ref) <= 1e-14 * mag)
    y0 = O.gemv_w4a16(w, s, None, x16.view(np.uint16))
    assert np.allclose(y - y0, b.astype(np.float64), rtol=0, atol=1e-15)


def test_gemv_w4a16_on_integer_x_equals_the_w4a8_gemv():
    """With x = fp16 of integer codes in [-127, 127] (exact in binary16) and
    s^x = 1, the float-unpack GEMV and the integer-dot GEMV compute the same
    sum: y agrees exactly."""
    N, K = 9, 3584
    q = I.uniform_int("pin/w4a16x/q", (N, K), -8, 7).numpy().astype(np.int8)
    w = O.pack_int4(q)
    s = I.normal("pin/w4a16x/s", N, 0.01).numpy()
    b = I.normal("pin/w4a16x/b", N, 0.01).numpy()
    qx = I.uniform_int("pin/w4a16x/x", K, -127, 127).numpy().astype(np.int8)
    x16 = qx.astype(np.float16)
    y16 = O.gemv_w4a16(w, s, b, x16.view(np.uint16))
    acc, y8 = O.gemv_w4a8(w, s, b, qx, np.float32(1.0))
    assert np.array_equal(y16, y8)
    assert np.array_equal(y16, s.astype(np.float64) * acc.astype(np.float64) + b.astype(np.float64))


def test_verify_matches_per_token_gemv():
    """[Ascend] 5: verifying M tokens streams the weights once; each token's
    column equals the single-token GEMV, and M = 1 is the GEMV itself."""
    N, K, M = 40, 256, 5
    W = I.normal("pin/ver/W", (N, K), 0.02).numpy()
    b = I.normal("pin/ver/b", N, 0.01).numpy()
    X = I.normal("pin/ver/X", (M, K)).numpy()
    w, s = O.prepare_int4_rowwise(W)
    qx, sx = O.quantize_act(X)
    acc, y = O.gemm_w4a8_verify(w, s, b, qx, sx)
    for m in range(M):
        a1, y1 = O.gemv_w4a8(w, s, b, qx[m], sx[m])
        assert np.array_equal(acc[m], a1) and np.array_equal(y[m], y1)
    a1, y1 = O.gemm_w4a8_verify(w, s, b, qx[:1], sx[:1])
    assert np.array_equal(a1[0], acc[0]) and np.array_equal(y1[0], y[0])


def test_errors_are_reported():
    with pytest.raises(O.OracleError):
        O.quantize_weights_int4_rowwise(np.array([[1.0, np.inf] + [0.0] * 6], np.float32))
    with pytest.raises(O.OracleError):
        O.quantize_weights_int4_group32(np.zeros((2, 48), np.float32))
    with pytest.raises(O.OracleError):   # -128 is outside the activation code range
        O.gemv_w4a8(np.zeros((1, 1), np.uint32), np.ones(1, np.float32), None,
                    np.array([-128] + [0] * 7, np.int8), 1.0)


# ------------------------------------------- producers fused with quant --
# The page names RMSNorm, SwiGLU and the residual add as the operators whose
# kernel boundaries could go ([Orin] "后续还能继续优化什么", items 1-2); the
# textbook definitions are checked here against numpy float64.
def _ulps(got, ref64):
    """|got - ref| in units of the fp32 spacing at ref (ref in float64)."""
    ref32 = ref64.astype(np.float32)
    return np.abs(got.astype(np.float64) - ref64) / np.spacing(np.abs(ref32)).astype(np.float64)


def _codes_tie_aware(q, v64):
    """Codes of fp32 values against round-half-even of the float64 values:
    equal, except within 1e-4 of a rounding tie, where either neighbour is
    accepted (the float64 reference and the fp32 decision may fall on either
    side)."""
    amax = np.abs(v64).max(axis=-1, keepdims=True)
    t = v64 / np.where(amax > 0, amax / 127.0, 1.0)
    near = np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-4
    exact = np.clip(np.round(t), -127, 127)
    ok = (q == exact) | (near & ((q == np.floor(t)) | (q == np.ceil(t))))
    return ok.all(), int(near.sum())


def test_exp_f32_within_two_ulps_of_numpy_float64():
    rng = np.random.default_rng(7)
    x = np.concatenate([np.linspace(-87.0, 88.0, 1_000_001).astype(np.float32),
                        rng.uniform(-87.0, 88.0, 200_000).astype(np.float32),
                        (np.arange(-120, 121) * np.float32(0.6931472)).astype(np.float32),
                        np.array([0.0, -0.0, 1e-30, -1e-30, 0.5, -0.5], np.float32)])
    x = x[(x > -87.0) & (x < 88.0)]
    got = O.exp_f32(x)
    assert _ulps(got, np.exp(x.astype(np.float64))).max() <= 2.0
    xs = np.sort(x)
    assert np.all(np.diff(O.exp_f32(xs)) >= 0)  # monotone
    assert O.exp_f32(np.float32([0.0]))[0] == 1.0
    assert O.exp_f32(np.float32([89.0, 200.0]))[0] == np.inf
    assert np.all(O.exp_f32(np.float32([-104.0, -300.0])) == 0.0)


def test_swiglu_vs_numpy_float64():
    rng = np.random.default_rng(11)
    M, I_ = 3, 4096
    g = (rng.standard_normal((M, I_)) * 2.0).astype(np.float32)
    u = rng.standard_normal((M, I_)).astype(np.float32)
    q, s, h = O.swiglu_quant(np.concatenate([g, u], axis=1))
    g64, u64 = g.astype(np.float64), u.astype(np.float64)
    h64 = g64 * u64 / (1.0 + np.exp(-g64))
    assert _ulps(h, h64).max() <= 4.0
    np.testing.assert_allclose(s, np.abs(h64).max(1) / 127.0, rtol=1e-6)
    ok, near = _codes_tie_aware(q, h64)
    assert ok and near < 10


def test_swiglu_closed_forms_and_permutation():
    rng = np.random.default_rng(12)
    I_ = 512
    # gate 0 (or up 0): h = 0, every code 0, s = 0
    for gu in (np.concatenate([np.zeros(I_), rng.standard_normal(I_)]),
               np.concatenate([rng.standard_normal(I_), np.zeros(I_)])):
        q, s, h = O.swiglu_quant(gu.astype(np.float32))
        assert s == 0.0 and not q.any() and not np.abs(h).any()
    # gate >= 30: e^-g < 2^-24, so 1 + e rounds to 1 and silu(g) = g exactly
    g = rng.uniform(30.0, 80.0, I_).astype(np.float32)
    u = rng.standard_normal(I_).astype(np.float32)
    _, _, h = O.swiglu_quant(np.concatenate([g, u]))
    assert np.array_equal(h, g * u)
    # pairs (g_i, u_i) permuted together permute h and the codes
    g = rng.standard_normal(I_).astype(np.float32)
    perm = rng.permutation(I_)
    q, s, h = O.swiglu_quant(np.concatenate([g, u]))
    qp, sp, hp = O.swiglu_quant(np.concatenate([g[perm], u[perm]]))
    assert sp == s and np.array_equal(hp, h[perm]) and np.array_equal(qp, q[perm])


def test_rmsnorm_vs_numpy_float64():
    rng = np.random.default_rng(13)
    M, K, eps = 3, 3584, 1e-6
    h = rng.standard_normal((M, K)).astype(np.float32)
    d = (rng.standard_normal((M, K)) * 0.5).astype(np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    q, s, h1, y = O.add_rmsnorm_quant(h, d, gamma, eps)
    assert np.array_equal(h1, h + d)  # numpy's IEEE fp32 add
    a = h1.astype(np.float64)
    y64 = a / np.sqrt((a * a).mean(1, keepdims=True) + eps) * gamma.astype(np.float64)
    assert _ulps(y, y64).max() <= 4.0
    np.testing.assert_allclose(s, np.abs(y64).max(1) / 127.0, rtol=1e-6)
    ok, near = _codes_tie_aware(q, y64)
    assert ok and near < 10
    # no residual: the same as a zero residual
    q0, s0, h10, y0 = O.add_rmsnorm_quant(h, None, gamma, eps)
    qz, sz, h1z, yz = O.add_rmsnorm_quant(h, np.zeros_like(h), gamma, eps)
    assert np.array_equal(q0, qz) and np.array_equal(s0, sz) and np.array_equal(y0, yz)


def test_rmsnorm_closed_forms():
    K = 64
    one = np.ones(K, np.float32)
    # a constant token normalises to +-1: every code is +-127
    for c in (3.0, -0.25, 1e-20):
        q, s, _, y = O.add_rmsnorm_quant(np.full(K, c, np.float32), None, one, 0.0)
        assert np.all(q == np.sign(c) * 127)
        assert np.all(np.abs(np.abs(y) - 1.0) <= 2.0 ** -23)
    # one spike a at index 5: r = 8 / |a|, y_5 = 8 sign(a), every other code 0
    for a in (5.0, -1e3):
        h = np.zeros(K, np.float32)
        h[5] = a
        q, s, _, y = O.add_rmsnorm_quant(h, None, one, 0.0)
        assert q[5] == np.sign(a) * 127 and np.count_nonzero(q) == 1
        assert abs(abs(float(y[5])) - 8.0) <= 8.0 * 2.0 ** -23
    # an all-zero token with eps = 0 normalises to zeros
    q, s, _, y = O.add_rmsnorm_quant(np.zeros(K, np.float32), None, one, 0.0)
    assert s == 0.0 and not q.any() and not y.any()


def test_rmsnorm_power_of_two_scale_invariance():
    """eps = 0: scaling h by 2^k scales the mean square by 4^k and r by 2^-k
    exactly, so y, s and the codes do not change."""
    rng = np.random.default_rng(14)
    h = rng.standard_normal(3584).astype(np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(3584)).astype(np.float32)
    q, s, _, y = O.add_rmsnorm_quant(h, None, gamma, 0.0)
    for k in (-20, 7, 30):
        qk, sk, h1k, yk = O.add_rmsnorm_quant(np.ldexp(h, k), None, gamma, 0.0)
        assert np.array_equal(qk, q) and sk == s and np.array_equal(yk, y)
        assert np.array_equal(h1k, np.ldexp(h, k))


# --------------------------------------------------- packed 6-bit lm_head --
# [Ascend] 3.2 gives the Q6_K sizes (256 weights in 210 bytes: 4-bit low and
# 2-bit high fields, an int8 scale per 16, an fp16 scale per 256); the
# quantiser and the array layout are this library's own.
def _golden_pairs(line):
    key, *items = line.split()
    return key, {int(a): int(b, 0) for a, b in (it.split(":") for it in items)}


def test_q6k_layout_golden():
    lines = [l for l in open(os.path.join(ROOT, "tests", "golden", "q6k_layout.txt"), encoding="utf-8")
             if l.strip() and not l.startswith("#")]
    tab = dict(_golden_pairs(l) for l in lines)
    q = np.full((1, 256), -32, np.int8)
    for i, c in tab["codes"].items():
        q[0, i] = c
    ql, qh = O.pack_q6k(q)
    assert ql.shape == (1, 128) and qh.shape == (1, 64)
    exp_ql = np.zeros(128, np.uint8)
    exp_qh = np.zeros(64, np.uint8)
    for i, v in tab["ql"].items():
        exp_ql[i] = v
    for i, v in tab["qh"].items():
        exp_qh[i] = v
    assert np.array_equal(ql[0], exp_ql) and np.array_equal(qh[0], exp_qh)
    assert np.array_equal(O.unpack_q6k(ql, qh), q)
    # 128 + 64 bytes of codes, 16 scales, one fp16: 210 bytes per 256 weights
    assert ql.nbytes + qh.nbytes + 16 + 2 == 210


def test_q6k_pack_round_trip_and_range():
    q = I.uniform_int("pin/q6k/rt", (5, 512), -32, 31).numpy().astype(np.int8)
    ql, qh = O.pack_q6k(q)
    assert np.array_equal(O.unpack_q6k(ql, qh), q)
    # every byte pattern of the packed arrays is a valid code set
    rng = np.random.default_rng(3)
    ql = rng.integers(0, 256, (3, 256), dtype=np.uint8)
    qh = rng.integers(0, 256, (3, 128), dtype=np.uint8)
    assert np.array_equal(O.pack_q6k(O.unpack_q6k(ql, qh))[0], ql)
    assert np.array_equal(O.pack_q6k(O.unpack_q6k(ql, qh))[1], qh)
    bad = q.copy()
    bad[0, 0] = 32
    with pytest.raises(O.OracleError):
        O.pack_q6k(bad)


def _rne(v):
    return np.array([round(float(t)) for t in np.ravel(v)], np.float64).reshape(np.shape(v))


def test_q6k_quantiser_vs_numpy_brute_force_and_bounds():
    W = I.normal("pin/q6k/W", (4, 512), 0.02).numpy()
    W[1, 256:272] = 0.0                      # a zero sub-block
    W[2, 0:256] *= np.repeat(np.float32([1e-3, 1.0]), 128)  # tiny sub-blocks under a large one
    q, sc, d = O.quantize_weights_q6k(W)
    for j in range(4):
        for b in range(2):
            wb = W[j, 256 * b:256 * (b + 1)].reshape(16, 16)
            t = (np.abs(wb).max(1).astype(np.float32) / np.float32(31)).astype(np.float32)
            dh = np.float16(np.float32(t.max()) / np.float32(127))
            assert d[j, b] == dh.view(np.uint16)
            df = np.float32(dh)
            exp_sc = np.clip(_rne(t / df), 0, 127) if df > 0 else np.zeros(16)
            assert np.array_equal(sc[j, 16 * b:16 * (b + 1)], exp_sc.astype(np.int8))
            e = (df * exp_sc.astype(np.float32)).astype(np.float32)
            for s in range(16):
                if e[s] == 0:
                    assert not q[j, 256 * b + 16 * s:256 * b + 16 * s + 16].any()
                    continue
                exp_q = np.clip(_rne(wb[s] / e[s]), -32, 31)
                assert np.array_equal(q[j, 256 * b + 16 * s:256 * b + 16 * s + 16], exp_q.astype(np.int8))
                # reconstruction within half a step, and the largest weight near the top code
                assert np.all(np.abs(wb[s].astype(np.float64) - e[s] * exp_q) <= 0.5 * e[s] * (1 + 1e-6))
                assert np.abs(exp_q).max() >= 28
            # the sub-block with the largest scale uses (almost) the whole int8 range
            assert sc[j, 16 * b:16 * (b + 1)].max() >= 126 or df == 0
    assert not sc[1, 16:32][0] and not q[1, 256:272].any()


def test_q6k_gemv_vs_numpy_float64_dequantised_matmul():
    N, K = 9, 1536
    W = I.normal("pin/q6k/gW", (N, K), 0.02).numpy()
    q, sc, d = O.quantize_weights_q6k(W)
    ql, qh = O.pack_q6k(q)
    x16 = I.normal("pin/q6k/x", K, 1.0, dtype=__import__("torch").float16).numpy()
    y = O.gemv_q6k_f16(ql, qh, sc, d, x16.view(np.uint16))
    e = (d.view(np.float16).astype(np.float64)[:, :, None] *
         sc.reshape(N, K // 256, 16).astype(np.float64)).reshape(N, K // 16)
    Wd = np.repeat(e, 16, axis=1) * q.astype(np.float64)
    ref = Wd @ x16.astype(np.float64)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # and the dequantised weights stay within half a step of W
    step = np.repeat(e, 16, axis=1)
    assert np.all(np.abs(Wd - W) <= 0.5 * step * (1 + 1e-6) + (step == 0) * np.abs(W))


# ---------------------------------------------------- INT8-X (3,5,8) codec --
# "定長無損 INT8 壓縮與 Triton 融合解碼", sections 2.1-2.5.
def test_int8x_layout_golden():
    tab = {}
    for l in open(os.path.join(ROOT, "tests", "golden", "int8x_layout.txt"), encoding="utf-8"):
        if l.strip() and not l.startswith("#"):
            k, *v = l.split()
            tab[k] = [int(t, 0) for t in v]
    q = np.tile(np.array(tab["pattern"], np.int8), 64).reshape(1, 512)
    e = O.int8x_encode(q)
    assert [e["n1"], e["n2"], e["n3"]] == tab["counts"]
    for k in ("b1", "b2", "l1", "l2"):
        assert int(e[k][0]) == tab[k][0], k
    assert list(e["l3"][:4]) == tab["l3"]
    assert list(e["b1_blk"]) == tab["b1_blk"] and list(e["b2_blk"]) == tab["b2_blk"]
    assert np.array_equal(O.int8x_decode(e), q.ravel())


def test_int8x_lossless_round_trip_and_block_decode():
    rng = np.random.default_rng(21)
    for q in (rng.integers(-128, 128, (7, 1024), dtype=np.int8),       # every byte value
              rng.integers(-3, 4, (3, 512), dtype=np.int8),             # level 1 only
              np.full((2, 512), -128, np.int8),                          # level 3 only
              np.clip(np.round(rng.laplace(0, 4.3, (9, 3584))), -127, 127).astype(np.int8)):
        e = O.int8x_encode(q)
        assert np.array_equal(O.int8x_decode(e), q.ravel())
        for t0, cnt in ((0, 1), (511, 3), (e["n"] - 5, 5), (e["n"] // 2 + 7, 100)):
            assert np.array_equal(O.int8x_decode(e, t0, cnt), q.ravel()[t0:t0 + cnt])
        n1, n2, n3 = O.int8x_counts(q)
        a = np.abs(q.astype(np.int32))
        assert (n1, n2, n3) == (int((a <= 3).sum()), int(((a > 3) & (a <= 15)).sum()), int((a > 15).sum()))


def test_int8x_bit_accounting_reproduces_the_page():
    """Level shares of 55.5 / 40.4 / 4.1 % (section 2.1) give flags 1.445 and
    data 4.013 bit/w, 5.46 in total (section 2.3)."""
    q = np.concatenate([np.full(555, 2), np.full(404, -9), np.full(41, 77)]).astype(np.int8)
    e = O.int8x_encode(np.random.default_rng(5).permutation(q))
    n = e["n"]
    flags = (n + e["n2"] + e["n3"]) / n
    data = (3 * e["n1"] + 5 * e["n2"] + 8 * e["n3"]) / n
    assert abs(flags - 1.445) < 1e-12 and abs(data - 4.013) < 1e-12
    assert round(O.int8x_bits(e) / n, 2) == 5.46


def test_gemv_int8x_vs_numpy_integer_matmul():
    """The GEMV over the encoded tensor against numpy's int64 matmul of the
    original (not decoded) codes."""
    rng = np.random.default_rng(22)
    N, K = 11, 3584
    q = np.clip(np.round(rng.laplace(0, 4.3, (N, K))), -127, 127).astype(np.int8)
    q[3, :] = rng.integers(-128, 128, K)
    qx = rng.integers(-127, 128, K).astype(np.int8)
    acc, y = O.gemv_int8x(O.int8x_encode(q), qx, 0.0123, 0.0031)
    ref = q.astype(np.int64) @ qx.astype(np.int64)
    assert np.array_equal(acc, ref)
    np.testing.assert_allclose(y, float(np.float32(0.0031)) * float(np.float32(0.0123)) * ref, rtol=1e-15)


# ------------------------------------------------ binary32 epilogue, chain --
def _round_f32(q):
    """The binary32 value nearest to the rational q, ties to even (normal
    and subnormal range; no overflow here)."""
    from fractions import Fraction
    if q == 0:
        return np.float32(0.0)
    neg, q = q < 0, abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()   # 2^e <= q < 2^(e+2)
    if Fraction(2) ** e > q:
        e -= 1
    if Fraction(2) ** (e + 1) <= q:
        e += 1
    e = max(e, -126)
    scale = Fraction(2) ** (e - 23)
    m = q / scale
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = float(n * scale)                     # representable: exact in binary64 too
    return np.float32(-v if neg else v)


def test_epilogue_f32_is_one_rounding_of_the_exact_value():
    """y = fl32(s * a + b) with s = fl32(sW sx) and a = fl32(acc): checked bit
    for bit against the exact rational rounded once; the samples include
    cases where an unfused multiply-add, an unrounded s, or a dropped bias
    would give other bits, so each of those mistakes fails here."""
    from fractions import Fraction
    rng = np.random.default_rng(11)
    N = 4000
    sw = (np.abs(rng.standard_normal(N)) * 3e-3 + 1e-5).astype(np.float32)
    sx = np.float32(0.0213)
    acc = rng.integers(-(1 << 26), 1 << 26, N).astype(np.int32)
    acc[:200] = rng.integers(-3000, 3000, 200)
    b = (rng.standard_normal(N) * 0.01).astype(np.float32)
    y = O.epilogue_f32(sw, b, sx, acc)
    y0 = O.epilogue_f32(sw, None, sx, acc)
    unfused = unrounded = 0
    for j in range(N):
        s = np.float32(sw[j]) * sx
        a = np.float32(acc[j])
        exact = Fraction(float(s)) * Fraction(float(a)) + Fraction(float(b[j]))
        ref = _round_f32(exact)
        assert y[j].view(np.uint32) == ref.view(np.uint32), j
        assert y0[j].view(np.uint32) == _round_f32(Fraction(float(s)) * Fraction(float(a))).view(np.uint32), j
        unfused += np.float32(np.float32(s * a) + b[j]) != ref
        unrounded += _round_f32(Fraction(float(sw[j])) * Fraction(float(sx)) * Fraction(float(a))
                                + Fraction(float(b[j]))) != ref
    assert unfused > 0 and unrounded > 0
    assert (y != y0).any()


def test_chain_brute_force_tiny():
    """The chain's wiring against a brute force in Python: codes from the
    pinned activation quantiser, acc from numpy's integer matmul of the
    unpacked codes, y32 the exact rational rounded once, and each linear's
    activation the first K values of the previous y32."""
    from fractions import Fraction
    shapes = [(64, 32), (48, 64), (16, 32)]
    rng = np.random.default_rng(5)
    lins = []
    for N, K in shapes:
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        w, sw = O.prepare_int4_rowwise(W)
        b = (rng.standard_normal(N) * 0.01).astype(np.float32) if N != 48 else None
        lins.append((w, sw, b))
    x = rng.standard_normal(32).astype(np.float32)
    out = O.chain_w4a8(lins, x)
    for t, ((w, sw, b), (N, K)) in enumerate(zip(lins, shapes)):
        qx, sx = O.quantize_act(x)
        acc = O.unpack_int4(w).astype(np.int64) @ qx.astype(np.int64)
        y32 = np.array([_round_f32(Fraction(float(np.float32(sw[j]) * np.float32(sx)))
                                   * Fraction(float(np.float32(acc[j])))
                                   + (Fraction(float(b[j])) if b is not None else 0)) for j in range(N)],
                       dtype=np.float32)
        oq, osx, oacc, oy64, oy32 = out[t]
        assert np.array_equal(oq, qx) and np.float32(osx) == np.float32(sx), t
        assert np.array_equal(oacc.astype(np.int64), acc), t
        assert np.array_equal(oy32.view(np.uint32), y32.view(np.uint32)), t
        if t + 1 < len(shapes):
            x = y32[:shapes[t + 1][1]]


def test_plain_relative_error_by_hand():
    """rel_err_plain: rows below 1e-3 of the largest |y_ref| (and zeros) are
    left out; the rest give |y - y_ref| / |y_ref|, worked by hand."""
    y_ref = np.array([1000.0, -2.0, 0.5, 0.0])
    y = np.array([1000.5, -2.002, 0.6, 1.0])
    assert O.rel_err_plain(y, y_ref) == pytest.approx(1e-3, rel=1e-9)      # the -2 row; 0.5 is below 1
    assert O.rel_err_plain(y, y_ref, floor=1e-4) == pytest.approx(0.2, rel=1e-9)   # 0.5 now counts
    assert O.rel_err_plain(y[:1], y_ref[:1]) == pytest.approx(5e-4, rel=1e-9)
    assert O.rel_err_plain(np.zeros(3), np.zeros(3)) == 0.0
    assert O.rel_err_plain(np.zeros(0), np.zeros(0)) == 0.0
