"""GPU parity: every entry point against the CPU oracle, element by element.

Bars: bit-exact for integers (packed weights, codes, int32 accumulators) and
fp32 scales that decide codes; fp32 outputs within 1e-5 relative error, the
error taken relative to the row's magnitude before cancellation (for a
per-row GEMV |sW sx acc| + |b|).  Inputs come from the seeded generator and
the same buffers feed both sides.
"""
import numpy as np
import pytest
import torch

import bit_quantized_decode_quantize_amd as bqd
import oracle as O
import parity_log as P
from bit_quantized_decode_quantize_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-5


def u32(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def npy(t):
    return t.detach().cpu().numpy()


def f16bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def sync():
    torch.cuda.synchronize()


def rel_err(y, y_ref, mag):
    y = np.asarray(y, np.float64)
    d = np.abs(y - y_ref)
    m = np.asarray(mag, np.float64)
    return np.where(m > 0, d / np.where(m > 0, m, 1.0), np.where(d > 0, np.inf, 0.0))


# ------------------------------------------------------ activation quant --
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
@pytest.mark.parametrize("K", [32, 64, 1536, 3584, 4096, 4128, 18944, 32768, 32800, 65536])
def test_quantize_act_bit_exact(K, dtype):
    """fp32 tokens up to 32768 values take the register-held producers'
    quantiser (1, 2, 4 or 8 items per thread), longer ones and fp16 the
    two-pass kernel: the same codes and scales either way."""
    M = 4
    x = I.normal(f"gpu/act/{K}", (M, K), 1.0, device=DEV, dtype=dtype)
    x[0] = I.with_outliers(x[0].float(), f"gpu/act/{K}/o").to(dtype)
    x[1] = x[1] * (1e-3 if dtype == torch.float16 else 1e-30)   # tiny magnitudes
    x[2] = 0                                                    # all-zero token
    x[3, K // 2] = -50.0                                        # negative maximum
    qx, sx = bqd.quantize_act(x)
    sync()
    qr, sr = O.quantize_act(npy(x))
    assert np.array_equal(npy(sx).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(npy(qx), qr)
    assert npy(qx)[3, K // 2] == -127 and not npy(qx)[2].any()


def test_quantize_act_rne_golden(golden):
    g = golden("act_quant_rne.txt")
    x = torch.zeros(32, dtype=torch.float32)
    vals = [float(v) for v in g["x"].split()]
    x[:len(vals)] = torch.tensor(vals)
    qx, sx = bqd.quantize_act(x.to(DEV))
    sync()
    assert float(npy(sx)[0]) == float(g["s"])
    assert list(npy(qx)[:len(vals)]) == [int(v) for v in g["q"].split()]


def _near_tie_vector(amax):
    """Values whose quotient by s = fl(amax/127) lies within a few ulps of
    every half-integer k + 1/2, |k| <= 126, plus amax itself."""
    a = np.float32(amax)
    s = np.float32(a / np.float32(127.0))
    vals = [a]
    for k in range(-126, 126):
        t = np.float32((k + 0.5) * np.float64(s))
        for j in range(-3, 4):
            v = t
            for _ in range(abs(j)):
                v = np.nextafter(v, np.float32(np.inf if j > 0 else -np.inf), dtype=np.float32)
            vals.append(v)
    vals = np.array(vals, np.float32)
    vals = vals[np.abs(vals) <= a]
    pad = (-vals.size) % 32
    return np.concatenate([vals, np.zeros(pad, np.float32)])


@pytest.mark.parametrize("amax", [100.0, 1.0, 3.0e-3, 7.77e5])
def test_quantize_act_near_ties_bit_exact(amax):
    """The reciprocal route must fall back to the exact quotient near ties."""
    x = _near_tie_vector(amax)
    qr, sr = O.quantize_act(x)
    xt = torch.from_numpy(x).to(DEV)
    qx, sx = bqd.quantize_act(xt)
    sync()
    assert npy(sx)[0] == sr and np.array_equal(npy(qx), qr)
    K = x.size
    w = torch.zeros((1, K // 8), dtype=torch.int32, device=DEV)
    _, qf, sf = bqd.linear_w4a8(w, torch.ones(1, device=DEV), None, xt, want_q=True)
    sync()
    assert npy(sf)[0] == sr and np.array_equal(npy(qf), qr)


def test_quantize_act_empty_is_noop():
    x = torch.zeros((0, 64), device=DEV)
    qx, sx = bqd.quantize_act(x)
    sync()
    assert qx.numel() == 0 and sx.numel() == 0


# ------------------------------------------------------- weight quant --
@pytest.mark.parametrize("N,K", [(1, 32), (7, 96), (129, 3584), (33, 18944)])
def test_quantize_weights_int4_rowwise_bit_exact(N, K):
    W = I.normal(f"gpu/wq/{N}/{K}", (N, K), 0.02, device=DEV)
    if N > 3:
        W[2] = 0.0
        W[3, 5] = -1.0
    wq, sw = bqd.quantize_weights_int4_rowwise(W)
    sync()
    qr, sr = O.quantize_weights_int4_rowwise(npy(W))
    assert np.array_equal(npy(sw).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(u32(wq), O.pack_int4(qr))


@pytest.mark.parametrize("N,K", [(1, 32), (9, 1536), (70, 6144)])
def test_quantize_weights_group32_bit_exact(N, K):
    W = I.normal(f"gpu/wq32/{N}/{K}", (N, K), 0.02, device=DEV)
    if N > 2:
        W[1, 32:64] = 0.0                  # zero group
        W[2, 64:96] *= 1e-4                # fp16-subnormal group scale
    wq, s16 = bqd.quantize_weights_int4_group32(W)
    w8, s8 = bqd.quantize_weights_int8_group32(W)
    sync()
    qr, sr = O.quantize_weights_int4_group32(npy(W))
    assert np.array_equal(f16bits(s16), sr)
    assert np.array_equal(u32(wq), O.pack_int4(qr))
    q8r, s8r = O.quantize_weights_int8_group32(npy(W))
    assert np.array_equal(f16bits(s8), s8r)
    assert np.array_equal(npy(w8), q8r)


# --------------------------------------------------------------- GEMVs --
def _rand_gemv(N, K, tag):
    w = I.random_words(f"gpu/g/{tag}/w", (N, K // 8), device=DEV)
    qx = I.uniform_int(f"gpu/g/{tag}/x", K, -127, 127, device=DEV, dtype=torch.int8)
    sw = I.normal(f"gpu/g/{tag}/s", N, 0.003, device=DEV).abs() + 1e-4
    b = I.normal(f"gpu/g/{tag}/b", N, 0.01, device=DEV)
    sx = torch.tensor([0.0421], device=DEV)
    return w, qx, sw, b, sx


def _check_rowwise(y, acc, w, sw, b, qx, sx):
    bb = None if b is None else npy(b)
    acc_r, y_r = O.gemv_w4a8(u32(w), npy(sw), bb, npy(qx), float(npy(sx)[0]))
    assert np.array_equal(npy(acc), acc_r)
    P.check_rowwise(f"N={y.numel()} K={npy(qx).size}", npy(y), y_r, npy(sw), npy(sx)[0], acc_r, bb, TOL)


GEMV_SHAPES = [(1, 32), (17, 64), (64, 96), (333, 3584), (3584, 3584), (130, 18944),
               (1000, 1536), (77, 2048), (200, 6144)]


@pytest.mark.parametrize("N,K", GEMV_SHAPES)
def test_gemv_w4a8_random_codes(N, K):
    w, qx, sw, b, sx = _rand_gemv(N, K, f"{N}/{K}")
    y, acc = bqd.gemv_w4a8(w, sw, b, qx, sx, acc=True)
    sync()
    _check_rowwise(y, acc, w, sw, b, qx, sx)
    y0, acc0 = bqd.gemv_w4a8(w, sw, None, qx, sx, acc=True)       # no bias
    sync()
    _check_rowwise(y0, acc0, w, sw, None, qx, sx)


@pytest.mark.parametrize("N,K", [(333, 3584), (130, 18944), (45, 32)])
def test_gemv_w4a8_every_config(N, K):
    w, qx, sw, b, sx = _rand_gemv(N, K, f"cfg/{N}/{K}")
    acc_r, _ = O.gemv_w4a8(u32(w), npy(sw), npy(b), npy(qx), float(npy(sx)[0]))
    for r in (1, 2, 4, 8):
        for L in (16, 32, 64):
            y, acc = bqd.gemv_w4a8(w, sw, b, qx, sx, acc=True, r=r, lanes_per_row=L)
            sync()
            assert np.array_equal(npy(acc), acc_r), (r, L)


@pytest.mark.parametrize("K", [3584, 18944])
def test_gemv_int32_bound_golden(golden, K):
    """All codes -8 against all -127 reach the page's bound 1016 K exactly."""
    g = golden("int32_bound.txt")
    N = 40
    w = torch.full((N, K // 8), 0x88888888 - (1 << 32), dtype=torch.int32, device=DEV)
    qx = torch.full((K,), -127, dtype=torch.int8, device=DEV)
    sw = torch.ones(N, device=DEV)
    sx = torch.ones(1, device=DEV)
    y, acc = bqd.gemv_w4a8(w, sw, None, qx, sx, acc=True)
    sync()
    assert np.all(npy(acc) == int(g["max_term"]) * K)
    if K == int(g["hidden"]):
        assert np.all(npy(acc) == int(g["row_bound"]))
    y, acc = bqd.gemv_w4a8(w, sw, None, -qx, sx, acc=True)
    sync()
    assert np.all(npy(acc) == -int(g["max_term"]) * K)


def test_gemv_empty_rows_is_noop():
    w = torch.zeros((0, 8), dtype=torch.int32, device=DEV)
    y = bqd.gemv_w4a8(w, torch.zeros(0, device=DEV), None, torch.zeros(64, dtype=torch.int8, device=DEV),
                      torch.ones(1, device=DEV))
    sync()
    assert y.numel() == 0


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_linear_w4a8_single_gemv_config(dtype):
    """The single Q-projection GEMV workload at full size, end to end on the
    device: weight quantisation, fused activation quantisation, GEMV."""
    d = I.single_gemv_inputs(seed=0, device=DEV)
    W, x, b = d["W"], d["x"].to(dtype), d["b"]
    wq, sw = bqd.quantize_weights_int4_rowwise(W)
    y, qx, sx, acc = bqd.linear_w4a8(wq, sw, b, x, want_q=True, want_acc=True)
    sync()
    wr, sr = O.prepare_int4_rowwise(npy(W))
    qxr, sxr, accr, yr = O.linear_w4a8(wr, sr, npy(b), npy(x))
    assert np.array_equal(u32(wq), wr) and np.array_equal(npy(sw), sr)
    assert np.array_equal(npy(qx), qxr) and npy(sx)[0] == sxr
    assert np.array_equal(npy(acc), accr)
    assert O.rel_err_rowwise(npy(y), yr, sr, sxr, accr, npy(b)).max() <= TOL


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
@pytest.mark.parametrize("K", [32, 1536, 8192, 8224, 24576, 65536])
def test_linear_w4a8_prologue_paths(K, dtype):
    """The fused prologue's two routes: up to K = 8192 the activation is held
    in registers (8192 fills them exactly), above it the two passes run in
    batches of 4 groups per thread (8224: a ragged last batch; 65536: the
    largest K).  Codes, s^x and accumulators bit-exact, per-row and group-32;
    1 % of x scaled by 20 so that the max sits anywhere."""
    N = 40
    x = I.with_outliers(I.normal(f"gpu/prol/{K}/x", K, 1.0, device=DEV), f"gpu/prol/{K}/o").to(dtype)
    w, _, sw, b, _ = _rand_gemv(N, K, f"prol/{K}")
    y, qx, sx, acc = bqd.linear_w4a8(w, sw, b, x, want_q=True, want_acc=True)
    sync()
    qxr, sxr = O.quantize_act(npy(x))
    assert np.array_equal(npy(qx), qxr) and npy(sx)[0] == sxr
    accr, yr = O.gemv_w4a8(u32(w), npy(sw), npy(b), qxr, float(sxr))
    assert np.array_equal(npy(acc), accr)
    assert O.rel_err_rowwise(npy(y), yr, npy(sw), sxr, accr, npy(b)).max() <= TOL
    s16 = I.normal(f"gpu/prol/{K}/s16", (N, K // 32), 0.01, device=DEV, dtype=torch.float16)
    yg, qg, sg, accg = bqd.linear_w4a8_group32(w, s16, None, x, want_q=True, want_acc=True)
    sync()
    assert np.array_equal(npy(qg), qxr) and npy(sg)[0] == sxr
    _check_group32(yg, accg, w, s16, None, qg, sg)


def test_linear_equals_quantize_then_gemv():
    """The fused prologue quantises exactly like quantize_act: same y bits."""
    w, _, sw, b, _ = _rand_gemv(1234, 18944, "fuse")
    x = I.swiglu_like("gpu/fuse/x", 18944, device=DEV)
    y1 = bqd.linear_w4a8(w, sw, b, x)
    qx, sx = bqd.quantize_act(x)
    y2 = bqd.gemv_w4a8(w, sw, b, qx, sx)
    sync()
    assert torch.equal(y1, y2)


# ------------------------------------------------------------ group-32 --
def _check_group32(y, accg, w, s16, b, qx, sx):
    bb = None if b is None else npy(b)
    accg_r, y_r = O.gemv_w4a8_group32(u32(w), f16bits(s16), bb, npy(qx), float(npy(sx)[0]))
    assert np.array_equal(npy(accg), accg_r)
    sg = f16bits(s16).view(np.float16).astype(np.float64)
    mag = float(npy(sx)[0]) * np.abs(sg * accg_r).sum(1) + (0 if bb is None else np.abs(bb))
    assert rel_err(npy(y), y_r, mag).max() <= TOL


@pytest.mark.parametrize("N,K", [(1, 32), (37, 96), (2048, 1536), (1536, 2048), (300, 6144)])
def test_gemv_w4a8_group32_random(N, K):
    w, qx, _, b, sx = _rand_gemv(N, K, f"g32/{N}/{K}")
    s16 = (I.normal(f"gpu/g32/{N}/{K}/s", (N, K // 32), 0.003, device=DEV).abs() + 1e-4).half()
    y, accg = bqd.gemv_w4a8_group32(w, s16, b, qx, sx, acc_g=True)
    sync()
    _check_group32(y, accg, w, s16, b, qx, sx)
    for r, L in ((1, 64), (8, 16), (2, 32)):
        y2, accg2 = bqd.gemv_w4a8_group32(w, s16, b, qx, sx, acc_g=True, r=r, lanes_per_row=L)
        sync()
        assert torch.equal(accg2, accg)
        _check_group32(y2, accg2, w, s16, b, qx, sx)


@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down"])
def test_linear_w4a8_group32_gemma_layer(name):
    N, K = dict((n, (a, k)) for n, a, k in I.gemma_layer_linears())[name]
    W = I.normal(f"gpu/gemma/{name}/W", (N, K), 0.02, device=DEV)
    x = I.linear_input("gpu/gemma", name, K, 0, DEV, torch.float16)
    wq, s16 = bqd.quantize_weights_int4_group32(W)
    y, qx, sx, accg = bqd.linear_w4a8_group32(wq, s16, None, x, want_q=True, want_acc=True)
    sync()
    wr, sr = O.prepare_int4_group32(npy(W))
    assert np.array_equal(u32(wq), wr) and np.array_equal(f16bits(s16), sr)
    qxr, sxr = O.quantize_act(npy(x))
    assert np.array_equal(npy(qx), qxr) and npy(sx)[0] == sxr
    _check_group32(y, accg, wq, s16, None, qx, sx)


# --------------------------------------------------------------- W8A16 --
@pytest.mark.parametrize("N,K", [(1, 32), (1001, 1536), (4096, 1536), (64, 4096)])
def test_gemv_w8a16_group32(N, K):
    q = I.uniform_int(f"gpu/w8/{N}/{K}/q", (N, K), -32, 31, device=DEV, dtype=torch.int8)
    q[0, :2] = torch.tensor([-32, 31], dtype=torch.int8)
    s16 = (I.normal(f"gpu/w8/{N}/{K}/s", (N, K // 32), 0.002, device=DEV).abs() + 1e-5).half()
    x16 = I.normal(f"gpu/w8/{N}/{K}/x", K, 1.0, device=DEV, dtype=torch.float16)
    yr = O.gemv_w8a16_group32(npy(q), f16bits(s16), f16bits(x16))
    sg = f16bits(s16).view(np.float16).astype(np.float64)
    ax = np.abs(f16bits(x16).view(np.float16).astype(np.float64))
    mag = (np.abs(npy(q)).astype(np.float64).reshape(N, -1, 32) * ax.reshape(-1, 32)).sum(2)
    mag = (sg * mag).sum(1)
    for r, L in ((0, 0), (1, 64), (8, 16), (4, 32)):
        y = bqd.gemv_w8a16_group32(q, s16, x16, r=r, lanes_per_row=L)
        sync()
        assert rel_err(npy(y), yr, mag).max() <= TOL, (r, L)


def test_gemv_w8a16_lm_head_codes_from_weights():
    N, K = 3000, 1536
    W = I.normal("gpu/w8lm/W", (N, K), 0.02, device=DEV)
    x16 = I.normal("gpu/w8lm/x", K, 1.0, device=DEV, dtype=torch.float16)
    w8, s16 = bqd.quantize_weights_int8_group32(W)
    y = bqd.gemv_w8a16_group32(w8, s16, x16)
    sync()
    q, s = O.quantize_weights_int8_group32(npy(W))
    assert np.array_equal(npy(w8), q) and np.array_equal(f16bits(s16), s)
    yr = O.gemv_w8a16_group32(q, s, f16bits(x16))
    sg = s.view(np.float16).astype(np.float64)
    ax = np.abs(f16bits(x16).view(np.float16).astype(np.float64))
    mag = (sg * (np.abs(q).astype(np.float64).reshape(N, -1, 32) * ax.reshape(-1, 32)).sum(2)).sum(1)
    assert rel_err(npy(y), yr, mag).max() <= TOL


# --------------------------------------------------- W4A16 comparison --
@pytest.mark.parametrize("N,K", [(1, 32), (37, 96), (3584, 3584), (300, 18944), (16389, 64)])
def test_gemv_w4a16(N, K):
    """Float-unpack GEMV against the oracle: random words (every nibble,
    -8 included) and fp16 x; every (r, lanes) configuration (N = 16389: the
    automatic two-rows-per-wave shape with a ragged last tile)."""
    w, _, sw, b, _ = _rand_gemv(N, K, f"w4a16/{N}/{K}")
    x16 = I.normal(f"gpu/w4a16/{N}/{K}/x", K, 1.0, device=DEV, dtype=torch.float16)
    yr = O.gemv_w4a16(u32(w), npy(sw), npy(b), f16bits(x16))
    q = np.abs(O.unpack_int4(u32(w))).astype(np.float64)
    mag = np.abs(npy(sw)).astype(np.float64) * (q @ np.abs(npy(x16).astype(np.float64))) + np.abs(npy(b))
    for r, L in ((0, 0), (1, 16), (2, 32), (4, 64), (8, 16)):
        y = bqd.gemv_w4a16(w, sw, b, x16, r=r, lanes_per_row=L)
        sync()
        assert rel_err(npy(y), yr, mag).max() <= TOL, (r, L)
    y0 = bqd.gemv_w4a16(w, sw, None, x16)
    sync()
    yr0 = O.gemv_w4a16(u32(w), npy(sw), None, f16bits(x16))
    assert rel_err(npy(y0), yr0, mag).max() <= TOL


def test_gemv_w4a16_integer_x_equals_w4a8():
    """x = fp16 of the int8 codes and s^x = 1: the float route reproduces the
    integer-dot GEMV (fp32 sums of integers below 2^24 are exact)."""
    N, K = 512, 3584
    w, qx, sw, b, _ = _rand_gemv(N, K, "w4a16int")
    one = torch.ones(1, device=DEV)
    y8, acc = bqd.gemv_w4a8(w, sw, b, qx, one, acc=True)
    y16 = bqd.gemv_w4a16(w, sw, b, qx.to(torch.float16))
    sync()
    assert np.abs(npy(acc)).max() < 2 ** 24
    assert torch.equal(y8, y16)


# ------------------------------------------------------- general K path --
@pytest.mark.parametrize("N,K", [(7, 8), (33, 40), (64, 104), (300, 3592), (5, 65544), (3, 2113664)])
def test_general_k_path(N, K):
    """K % 8 == 0 outside the fast kernels' range (K % 32 != 0, or more codes
    than BQD_MAX_K, up to the int32 bound): quantize_act, gemv_w4a8,
    linear_w4a8 (fp32 and fp16 x) and the automatic verify take the general
    kernel.  Codes, s^x and acc bit-exact against the oracle, y within
    tolerance, the verify's token rows equal to the one-token GEMV."""
    w, qx, sw, b, sx = _rand_gemv(N, K, f"anyk/{N}/{K}")
    g, acc = bqd.gemv_w4a8(w, sw, b, qx, sx, acc=True, r=2, lanes_per_row=16)  # r, lanes not used here
    sync()
    _check_rowwise(g, acc, w, sw, b, qx, sx)
    X = I.normal(f"gpu/anyk/{K}/X", (2, K), 1.0, device=DEV)
    for xin in (X[1].contiguous(), X[1].to(torch.float16)):
        y, q, s1, a = bqd.linear_w4a8(w, sw, b, xin, want_q=True, want_acc=True)
        sync()
        qo, so = O.quantize_act(npy(xin))
        assert np.array_equal(npy(q), qo) and npy(s1)[0] == so
        acc_r, y_r = O.gemv_w4a8(u32(w), npy(sw), npy(b), qo, float(so))
        assert np.array_equal(npy(a), acc_r)
        P.check_rowwise(f"linear {xin.dtype} N={N} K={K}", npy(y), y_r, npy(sw), so, acc_r, npy(b), TOL)
    QX, SX = bqd.quantize_act(X)
    sync()
    qo, so = O.quantize_act(npy(X))
    assert np.array_equal(npy(QX), qo) and np.array_equal(npy(SX), so)
    Y, A = bqd.gemm_w4a8_verify(w, sw, b, QX, SX, acc=True)
    sync()
    acc_r, y_r = O.gemm_w4a8_verify(u32(w), npy(sw), npy(b), qo, so)
    assert np.array_equal(npy(A), acc_r)
    for m in range(2):
        P.check_rowwise(f"verify token {m}", npy(Y)[m], y_r[m], npy(sw), so[m], acc_r[m], npy(b), TOL)
        y1 = bqd.gemv_w4a8(w, sw, b, QX[m].clone(), SX[m:m + 1].clone())  # a copy: 16-byte aligned
        sync()
        assert torch.equal(y1, Y[m])


# -------------------------------------------------------------- verify --
@pytest.mark.parametrize("impl", [0, 1, 2, 3])
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("N,K", [(200, 3584), (150, 18944), (33, 64), (70, 96)])
def test_gemm_w4a8_verify(M, N, K, impl):
    """impl 1: dot-product kernel; impl 2: matrix cores (K split over 16
    waves here: few rows; K = 64 / 96 leave lane groups without a chunk);
    impl 3: matrix cores in balanced blocks (few tiles: K split over
    workgroups, partials through the workspace); impl 0: automatic (the
    GEMV kernel for one token)."""
    w, _, sw, b, _ = _rand_gemv(N, K, f"ver/{N}/{K}")
    X = I.normal(f"gpu/ver/{M}/{K}/X", (M, K), 1.0, device=DEV)
    qx, sx = bqd.quantize_act(X)
    y, acc = bqd.gemm_w4a8_verify(w, sw, b, qx, sx, acc=True, impl=impl)
    sync()
    acc_r, y_r = O.gemm_w4a8_verify(u32(w), npy(sw), npy(b), npy(qx), npy(sx))
    assert np.array_equal(npy(acc), acc_r)
    for m in range(M):
        P.check_rowwise(f"token {m}", npy(y)[m], y_r[m], npy(sw), npy(sx)[m], acc_r[m], npy(b), TOL)
    # token m's column equals the single-token GEMV bit for bit
    for m in (0, M - 1):
        y1 = bqd.gemv_w4a8(w, sw, b, qx[m].contiguous(), sx[m:m + 1].contiguous())
        sync()
        assert torch.equal(y1, y[m])


@pytest.mark.parametrize("M", [4, 16])
@pytest.mark.parametrize("N,K", [(32770, 64), (16400, 256), (8200, 128), (4100, 160)])
def test_gemm_w4a8_verify_mfma_row_tilings(M, N, K):
    """Matrix-core verify on a 256-CU device: one wave per 16-row tile
    (N = 32770), 2, 4 and 8 waves per tile (N = 16400, 8200, 4100; the small
    shapes of the test above take 16); ragged last tile.  Bit-exact acc
    against the oracle, y within tolerance, y identical to the dot-product
    kernel."""
    w, _, sw, b, _ = _rand_gemv(N, K, f"vermf/{N}/{K}")
    X = I.normal(f"gpu/vermf/{M}/{K}/X", (M, K), 1.0, device=DEV)
    qx, sx = bqd.quantize_act(X)
    y, acc = bqd.gemm_w4a8_verify(w, sw, b, qx, sx, acc=True, impl=2)
    y1 = bqd.gemm_w4a8_verify(w, sw, b, qx, sx, impl=1)
    y3, acc3 = bqd.gemm_w4a8_verify(w, sw, b, qx, sx, acc=True, impl=3)
    sync()
    acc_r, y_r = O.gemm_w4a8_verify(u32(w), npy(sw), npy(b), npy(qx), npy(sx))
    assert np.array_equal(npy(acc), acc_r)
    assert np.array_equal(npy(acc3), acc_r)
    for m in range(M):
        P.check_rowwise(f"token {m}", npy(y)[m], y_r[m], npy(sw), npy(sx)[m], acc_r[m], npy(b), TOL)
    assert torch.equal(y, y1)
    assert torch.equal(y3, y1)


@pytest.mark.parametrize("M,N,K", [(16, 3584, 18944), (2, 100, 65536), (16, 4100, 2048), (5, 17, 32)])
def test_verify_blocks_workspace(M, N, K):
    """The balanced matrix-core verify at shapes whose K is split over
    workgroups (the down-shaped verify, a long K with few rows) or not: the
    workspace the binding hands over is zero again after each call, calls in
    a row give the same bits, a caller's own zeroed workspace works too, and
    acc equals the oracle's."""
    w, _, sw, b, _ = _rand_gemv(N, K, f"vbws/{N}/{K}")
    X = I.normal(f"gpu/vbws/{M}/{K}/X", (M, K), 1.0, device=DEV)
    qx, sx = bqd.quantize_act(X)
    need = bqd.lib().gemm_w4a8_verify_workspace_bytes(M, N, K)
    ws = bqd.verify_workspace(M, N, K, DEV)
    assert (ws is None) == (need == 0)
    outs = []
    for _ in range(3):
        outs.append(bqd.gemm_w4a8_verify(w, sw, b, qx, sx, acc=True, impl=3))
        sync()
        if ws is not None:
            assert int(ws.abs().max()) == 0   # the whole workspace is zero again
    if need:
        own = torch.zeros(need // 4 + 64, dtype=torch.int32, device=DEV)
        outs.append(bqd.gemm_w4a8_verify(w, sw, b, qx, sx, acc=True, impl=3, workspace=own))
        sync()
        assert int(own.abs().max()) == 0    # counts and partials are zero again
        with pytest.raises(bqd.BQDError):
            bqd.gemm_w4a8_verify(w, sw, b, qx, sx, impl=3, workspace=own[:16])
    for y, acc in outs[1:]:
        assert torch.equal(y, outs[0][0]) and torch.equal(acc, outs[0][1])
    acc_r, y_r = O.gemm_w4a8_verify(u32(w), npy(sw), npy(b), npy(qx), npy(sx))
    assert np.array_equal(npy(outs[0][1]), acc_r)
    for m in (0, M - 1):
        P.check_rowwise(f"token {m}", npy(outs[0][0])[m], y_r[m], npy(sw), npy(sx)[m], acc_r[m], npy(b), TOL)


# -------------------------------------------------------- layer launcher --
def test_layer_forward_fused_rows_equal_separate_linears():
    """Concatenated q/k/v rows run as one linear give the same bits as the
    three linears run on their row slices."""
    from bit_quantized_decode_quantize_amd import decode_stream as DS
    W = DS.linear_weight_fp32("gpu/layer", "qkv", 0, DEV)
    b = DS.layer_biases("gpu/layer", 0, DEV)["qkv"]
    x = I.normal("gpu/layer/x", 3584, 1.0, device=DEV)
    wq, sw = bqd.quantize_weights_int4_rowwise(W)
    y = torch.empty(4608, device=DEV)
    bqd.layer_w4a8_forward([bqd.make_linear(wq, sw, b)], [x], [y])
    parts = []
    for lo, hi in ((0, 3584), (3584, 4096), (4096, 4608)):
        parts.append(bqd.linear_w4a8(wq[lo:hi], sw[lo:hi], b[lo:hi], x))
    sync()
    assert torch.equal(y, torch.cat(parts))


@pytest.mark.parametrize("persistent", [False, True])
def test_qwen_layer_full_size_sampled(persistent):
    """One Qwen2-7B-shaped layer at full size, through layer_w4a8_forward (one
    launch per linear) or the persistent pass; 300 sampled rows per linear
    (plus the first and last) against the oracle."""
    from bit_quantized_decode_quantize_amd import decode_stream as DS
    s = DS.QwenW4A8Stream(layers=1, lm_head=False, device=DEV, persistent=persistent)
    s.step()
    sync()
    for d in s.linears:
        N, K = d["N"], d["K"]
        rows = torch.cat([torch.tensor([0, N - 1]),
                          I.distinct_indices(f"gpu/sample/{d['name']}", N, 300)]).unique()
        Wr = npy(s.fp32_rows(d, rows))
        wr, sr = O.prepare_int4_rowwise(Wr)
        idx = rows.to(DEV)
        assert np.array_equal(u32(d["wq"][idx]), wr)
        assert np.array_equal(npy(d["sw"][idx]), sr)
        br = npy(d["b"][idx])
        qxr, sxr, accr, yr = O.linear_w4a8(wr, sr, br, npy(d["x"]))
        P.check_rowwise(d["name"], npy(d["y"][idx]), yr, sr, sxr, accr, br, TOL)


# ------------------------------------------------------- persistent pass --
PASS_SHAPES = [(4608, 3584), (3584, 3584), (300, 18944), (17, 64), (1, 32), (5000, 1536), (37888, 3584)]


def _pass_fixture(dtype=torch.float32, tag="pass"):
    lins, xs, ys, parts = [], [], [], []
    for i, (N, K) in enumerate(PASS_SHAPES):
        W = I.normal(f"gpu/{tag}/{i}/W", (N, K), 0.02, device=DEV)
        wq, sw = bqd.quantize_weights_int4_rowwise(W)
        b = I.normal(f"gpu/{tag}/{i}/b", N, 0.01, device=DEV) if i % 2 == 0 else None
        x = I.normal(f"gpu/{tag}/{i}/x", K, 1.0, device=DEV, dtype=dtype)
        y = torch.full((N,), float("nan"), device=DEV)
        lins.append(bqd.make_linear(wq, sw, b))
        xs.append(x)
        ys.append(y)
        parts.append((wq, sw, b, x))
    return lins, xs, ys, parts


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_decode_pass_equals_per_linear_launches(dtype):
    lins, xs, ys, parts = _pass_fixture(dtype, f"pass{dtype}")
    p = bqd.DecodePass(lins, xs, ys)
    assert p.sources() == [-1] * len(lins)  # no activation is an output of the pass
    ref = [bqd.linear_w4a8(wq, sw, b, x) for wq, sw, b, x in parts]
    for rep in range(3):                     # the workspace carries over between passes
        for y in ys:
            y.fill_(float("nan"))
        p.run()
        sync()
        assert p.error_word() == 0
        for i, (y, yr) in enumerate(zip(ys, ref)):
            assert torch.equal(y, yr), (rep, i)
    # and against the oracle on one linear, end to end
    wq, sw, b, x = parts[2]
    qxr, sxr, accr, yr = O.linear_w4a8(u32(wq), npy(sw), npy(b), npy(x))
    assert O.rel_err_rowwise(npy(ys[2]), yr, npy(sw), sxr, accr, npy(b)).max() <= TOL


CHAIN_SHAPES = [(2048, 1024), (1024, 2048), (4096, 1024), (1024, 4096), (1024, 1024), (2944, 1024),
                (1024, 2944), (8192, 1024), (1024, 8192), (24576, 1024), (1000, 24576)]

XCH_BASE = 64 + 1024 * 16   # exchange words start after the error line and the epoch lines


def _chain(tag, shapes, oracle_chain=False):
    """Linears chained as a decoder chains them: linear i+1 reads the first
    K values of linear i's output (distinct buffers).  Returns the pass
    pieces, the same chain run one launch per linear, and (oracle_chain)
    the oracle's own run of the chain from the same fp32 weights, biases and
    first activation (drawn on the host, copied to the device)."""
    lins, parts, host = [], [], []
    for i, (N, K) in enumerate(shapes):
        W = I.normal(f"gpu/{tag}/{i}/W", (N, K), 0.02)
        b = I.normal(f"gpu/{tag}/{i}/b", N, 0.01) if i % 2 == 0 else None
        wq, sw = bqd.quantize_weights_int4_rowwise(W.to(DEV))
        bd = None if b is None else b.to(DEV)
        lins.append(bqd.make_linear(wq, sw, bd))
        parts.append((wq, sw, bd))
        host.append((W, b))
    x0h = I.normal(f"gpu/{tag}/x", shapes[0][1], 1.0)
    x0 = x0h.to(DEV)
    ys = [torch.full((N,), float("nan"), device=DEV) for N, _ in shapes]
    xs = [x0] + [ys[i - 1][:K] for i, (_, K) in enumerate(shapes) if i > 0]
    ref, xr = [], x0
    for i, ((N, K), (wq, sw, b)) in enumerate(zip(shapes, parts)):
        ref.append(bqd.linear_w4a8(wq, sw, b, xr))
        xr = ref[-1][:shapes[i + 1][1]] if i + 1 < len(shapes) else None
    sync()
    orc = None
    if oracle_chain:
        prepared = []
        for (W, b), (wq, sw, _) in zip(host, parts):
            w_r, s_r = O.prepare_int4_rowwise(W.numpy())
            assert np.array_equal(u32(wq), w_r) and np.array_equal(npy(sw), s_r)
            prepared.append((w_r, s_r, None if b is None else b.numpy()))
        orc = (prepared, O.chain_w4a8(prepared, x0h.numpy()))
    return lins, parts, xs, ys, ref, orc


def test_decode_pass_chained():
    """A decoder's chain inside one pass, K up to the pass's largest: each
    linear reads what the previous one wrote, through the exchange.  Every
    output equals the oracle's own run of the chain bit for bit (the value
    handed on is decided in binary32 on both sides, so codes, accumulators
    and the binary32 y agree exactly) and lies within the tolerance of the
    binary64 y; it also equals the chain launched one linear at a time.
    After each of three passes the exchange set the pass used holds every
    read output as ~bits(y), and the other set is all zero (ready for the
    next pass)."""
    lins, parts, xs, ys, ref, (prepared, orc) = _chain("chain", CHAIN_SHAPES, oracle_chain=True)
    for i, (yr, (qx, sx, acc, y64, y32)) in enumerate(zip(ref, orc)):
        w_r, s_r, b_r = prepared[i]
        assert np.array_equal(npy(yr).view(np.uint32), y32.view(np.uint32)), i
        P.check_rowwise(f"linear {i}", npy(yr), y64, s_r, sx, acc, b_r, TOL)
    p = bqd.DecodePass(lins, xs, ys)
    src = p.sources()
    assert src[0] == -1 and all(v >= 0 for v in src[1:])
    words = (p.sync.numel() - XCH_BASE) // 2
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        p.run()
        sync()
        assert p.error_word() == 0
        for i, (y, yr) in enumerate(zip(ys, ref)):
            assert torch.equal(y, yr), (rep, i)
        w = p.sync.cpu().numpy().view(np.uint32)
        epoch = int(w[64])
        assert epoch == rep + 1 and (w[64:64 + 16 * 1024:16][:_grid(p)] == epoch).all()
        cur = w[XCH_BASE + (epoch & 1) * words:][:words]
        old = w[XCH_BASE + ((epoch & 1) ^ 1) * words:][:words]
        assert not old.any()
        for i in range(len(lins) - 1):           # y[i] is read by linear i + 1
            o = src[i + 1]                        # x[i+1] = y[i][:K]: its words start y[i]'s
            yb = npy(ys[i]).view(np.uint32)
            assert np.array_equal(~cur[o:o + yb.size], yb), (rep, i)


def _grid(p):
    return int(p.desc[4:8].cpu().view(torch.int32).item())


def test_decode_pass_rejects_reused_buffers():
    """Workgroups run ahead of each other where no data dependency holds
    them, so a pass writes each output exactly once and never over an
    activation it reads: a chain through two reused buffers is refused."""
    shapes = CHAIN_SHAPES[:4]
    cap = max(max(N, K) for N, K in shapes)
    lins = []
    for i, (N, K) in enumerate(shapes):
        wq, sw = bqd.quantize_weights_int4_rowwise(I.normal(f"gpu/reuse/{i}/W", (N, K), 0.02, device=DEV))
        lins.append(bqd.make_linear(wq, sw, None))
    bufs = [torch.zeros(cap, device=DEV), torch.zeros(cap, device=DEV)]
    xs = [bufs[i % 2][:K] for i, (N, K) in enumerate(shapes)]
    ys = [bufs[(i + 1) % 2][:N] for i, (N, K) in enumerate(shapes)]
    with pytest.raises(bqd.BQDError) as e:
        bqd.DecodePass(lins, xs, ys)
    assert e.value.status == -2


def test_decode_pass_epochs_wrap_around():
    """Epoch words preset from the host to 2^32 - 1: the next two passes run
    as epochs 0 and 1 (the exchange sets alternate by parity across the
    wrap) with every output equal to the per-linear launches."""
    lins, parts, xs, ys, ref, _ = _chain("chainwrap", CHAIN_SHAPES[:5])
    p = bqd.DecodePass(lins, xs, ys)
    words = np.zeros(p.sync.numel(), dtype=np.uint32)
    words[64:64 + 16 * 1024:16] = 0xFFFFFFFF
    p.sync.copy_(torch.from_numpy(words.view(np.int32)).to(DEV))
    for rep in range(2):
        for y in ys:
            y.fill_(float("nan"))
        p.run()
        sync()
        assert p.error_word() == 0, rep
        for i, (y, yr) in enumerate(zip(ys, ref)):
            assert torch.equal(y, yr), (rep, i)
    out = p.sync.cpu().numpy().view(np.uint32)
    assert (out[64:64 + 16 * _grid(p):16] == 1).all()


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_decode_pass_at_the_largest_k(dtype):
    """Linears at the pass's largest K (its LDS holds K codes and 4K bytes of
    fp32 activation) between small ones, ragged row counts: every output
    equals the per-linear launch, one against the oracle."""
    K = bqd.BQD_MAX_PASS_K
    shapes = [(300, K), (1000, 32), (17, K), (4100, 64)]
    lins, xs, ys, parts = [], [], [], []
    for i, (N, Ki) in enumerate(shapes):
        W = I.normal(f"gpu/passmax/{i}/W", (N, Ki), 0.02, device=DEV)
        wq, sw = bqd.quantize_weights_int4_rowwise(W)
        b = I.normal(f"gpu/passmax/{i}/b", N, 0.01, device=DEV) if i % 2 == 0 else None
        x = I.normal(f"gpu/passmax/{i}/x", Ki, 1.0, device=DEV, dtype=dtype)
        lins.append(bqd.make_linear(wq, sw, b))
        xs.append(x)
        ys.append(torch.full((N,), float("nan"), device=DEV))
        parts.append((wq, sw, b, x))
    p = bqd.DecodePass(lins, xs, ys)
    assert p.max_k == K
    p.run()
    p.run()
    sync()
    assert p.error_word() == 0
    for i, ((wq, sw, b, x), y) in enumerate(zip(parts, ys)):
        assert torch.equal(y, bqd.linear_w4a8(wq, sw, b, x)), i
    wq, sw, b, x = parts[0]
    qxr, sxr, accr, yr = O.linear_w4a8(u32(wq), npy(sw), npy(b), npy(x))
    assert O.rel_err_rowwise(npy(ys[0]), yr, npy(sw), sxr, accr, npy(b)).max() <= TOL


def test_decode_pass_zero_activation_gives_the_bias():
    """A linear of the pass whose activation is all zero has s^x = 0, zero
    codes and y = b exactly (the degenerate case of the per-token scale);
    the linears around it are unaffected."""
    lins, xs, ys, parts = _pass_fixture(tag="passzero")
    xs[2].zero_()
    p = bqd.DecodePass(lins, xs, ys)
    p.run()
    sync()
    assert p.error_word() == 0
    wq, sw, b, x = parts[2]
    assert b is not None and torch.equal(ys[2], b)
    for i, ((wq, sw, b, x), y) in enumerate(zip(parts, ys)):
        assert torch.equal(y, bqd.linear_w4a8(wq, sw, b, x)), i


def test_pass_descriptors_keep_their_tensors():
    """Descriptors built from tensors nothing else refers to (a helper's
    locals) stay valid: the descriptor holds its tensors and the pass its
    descriptors, so new allocations cannot take their memory."""
    def build(i, N, K):
        W = I.normal(f"gpu/keep/{i}/W", (N, K), 0.02, device=DEV)
        wq, sw = bqd.quantize_weights_int4_rowwise(W)
        ref = bqd.linear_w4a8(wq, sw, None, x0[:K])
        return bqd.make_linear(wq, sw, None), ref
    x0 = I.normal("gpu/keep/x", 3584, 1.0, device=DEV)
    built = [build(i, N, K) for i, (N, K) in enumerate([(700, 3584), (300, 1536), (900, 3584)])]
    sync()
    lins, refs = [b[0] for b in built], [b[1] for b in built]
    ys = [torch.full((l.N,), float("nan"), device=DEV) for l in lins]
    p = bqd.DecodePass(lins, [x0[:l.K] for l in lins], ys)
    del lins, built
    junk = [torch.full((1 << 20,), 7, dtype=torch.int32, device=DEV) for _ in range(16)]  # reuse freed memory
    p.run()
    sync()
    assert p.error_word() == 0
    for y, r in zip(ys, refs):
        assert torch.equal(y, r)
    del junk


def test_decode_pass_wait_limit_sets_error_and_ends():
    """A one-round spin limit, set from the host, makes a wait give up at its
    first unanswered poll.  Linears 0..9 ([32, K_max] each) occupy
    workgroups 0..31 only, each staging a 96 KB activation per linear; the
    other workgroups have no rows there and go straight to linear 10, which
    reads linear 9's output, long before it can exist: their waits run out,
    bit 0 is set (bit 1 is not), and the kernel still ends.  A normal pass
    afterwards gives the outputs of one launch per linear."""
    K = bqd.BQD_MAX_PASS_K
    lins, xs, ys, parts = [], [], [], []
    for i in range(11):
        N, Ki = (32, K) if i < 10 else (4096, 32)
        wq, sw = bqd.quantize_weights_int4_rowwise(I.normal(f"gpu/passlim/{i}/W", (N, Ki), 0.02, device=DEV))
        lins.append(bqd.make_linear(wq, sw, None))
        ys.append(torch.full((N,), float("nan"), device=DEV))
        xs.append(I.normal(f"gpu/passlim/{i}/x", Ki, 1.0, device=DEV) if i < 10 else ys[9])
        parts.append((wq, sw))
    p = bqd.DecodePass(lins, xs, ys)
    assert p.sources()[:10] == [-1] * 10 and p.sources()[10] >= 0
    p.run(spin_limit=1)
    sync()
    assert p.error_word() == 1
    p.clear_error()
    p.run()
    sync()
    assert p.error_word() == 0
    for i in range(11):
        wq, sw = parts[i]
        assert torch.equal(ys[i], bqd.linear_w4a8(wq, sw, None, xs[i] if i < 10 else ys[9])), i


def test_qwen_stream_full_size_persistent_sampled():
    """The bench's workload and launch configuration: the full 28-layer
    stream + lm_head as one persistent pass; sampled rows of linears across
    the stream against the oracle, and every output equal to the
    per-linear launches."""
    from bit_quantized_decode_quantize_amd import decode_stream as DS
    s = DS.QwenW4A8Stream(layers=28, device=DEV, persistent=True)
    s.step()
    s.step()
    sync()
    assert s.pass_.error_word() == 0
    for k in (0, 1, 53, 54, 111, 112):      # L0 qkv/o, L13 gate_up/down, L27 down, lm_head
        d = s.linears[k]
        yr = bqd.linear_w4a8(d["wq"], d["sw"], d["b"], d["x"])
        sync()
        assert torch.equal(d["y"], yr), d["name"]
        N = d["N"]
        rows = torch.cat([torch.tensor([0, N - 1]),
                          I.distinct_indices(f"gpu/stream/{k}", N, 200)]).unique()
        Wr = npy(s.fp32_rows(d, rows))
        wr, sr = O.prepare_int4_rowwise(Wr)
        idx = rows.to(DEV)
        assert np.array_equal(u32(d["wq"][idx]), wr)
        br = None if d["b"] is None else npy(d["b"][idx])
        qxr, sxr, accr, y_r = O.linear_w4a8(wr, sr, br, npy(d["x"]))
        P.check_rowwise(f"linear {k} {d['name']}", npy(d["y"][idx]), y_r, sr, sxr, accr, br, TOL)
    # The same linears cut to 64 rows: the full pass's first 64 rows, bit
    # for bit.
    fp = s.cut_pass(64)
    fp.run()
    sync()
    assert fp.error_word() == 0
    for i, d in enumerate(s.linears):
        assert torch.equal(fp.outputs[i], d["y"][:64]), (i, d["name"])
    # The same 113 linears chained as a decoder chains them: each reads the
    # previous one's output (a prefix where the previous linear is wider,
    # e.g. QKV -> O); every output equals the chain launched one linear at a
    # time.
    p = s.chained_pass()
    ys = p.outputs
    for y in ys:
        y.fill_(float("nan"))
    src = p.sources()
    assert src[0] == -1 and all(v >= 0 for v in src[1:])
    p.run()
    p.run()
    sync()
    assert p.error_word() == 0
    xr = s.linears[0]["x"]
    for i, d in enumerate(s.linears):
        yr = bqd.linear_w4a8(d["wq"], d["sw"], d["b"], xr)
        assert torch.equal(ys[i], yr), (i, d["name"])
        xr = yr[:s.linears[i + 1]["K"]] if i + 1 < len(s.linears) else None
    sync()


def _g32_pass(tag, chained):
    """Two Gemma-shaped group-32 layers (QKV, O, gate/up, down) as one pass:
    fp16 activations written before the launch, or chained through fp32
    outputs (linear i+1 reads the first K values of linear i's output)."""
    lins, parts, xs, ys, xhost = [], [], [], [], []
    for l in range(2):
        for name, N, K in I.gemma_layer_linears():
            W = I.normal(f"gpu/{tag}/{l}/{name}/W", (N, K), 0.02)
            wq, s16 = bqd.quantize_weights_int4_group32(W.to(DEV))
            lins.append(bqd.make_linear(wq, s16, None))
            parts.append((W, wq, s16))
            ys.append(torch.full((N,), float("nan"), device=DEV))
            if not chained:
                xh = I.linear_input(f"gpu/{tag}/{l}", name, K, 0, "cpu", torch.float16)
                xhost.append(xh)
                xs.append(xh.to(DEV))
    if chained:
        xh = I.normal(f"gpu/{tag}/x0", parts[0][0].shape[1], 1.0)
        xhost.append(xh)
        xs = [xh.to(DEV)] + [ys[i - 1][:W.shape[1]] for i, (W, _, _) in enumerate(parts) if i > 0]
    return lins, parts, xs, ys, xhost


def _g32_oracle_first(parts, xhost, y):
    """The pass's first linear against the oracle run from the host's fp32
    weights and activation: packed words and scales equal, y within the
    tolerance of the magnitude before cancellation."""
    W, wq, s16 = parts[0]
    wr, sr = O.prepare_int4_group32(W.numpy())
    assert np.array_equal(u32(wq), wr) and np.array_equal(f16bits(s16), sr)
    xr = xhost[0].numpy()
    _, sxr, accr, yr = O.linear_w4a8_group32(wr, sr, None, xr)
    mag = float(sxr) * np.abs(sr.view(np.float16).astype(np.float64) * accr).sum(1)
    assert rel_err(npy(y), yr, mag).max() <= TOL


def test_decode_pass_group32_equals_per_linear_launches():
    """Group-32 linears ("在香橙派上跑 Gemma4 ..." section 3.1) in the pass, fp16
    activations: every output equals linear_w4a8_group32 bit for bit over
    three passes (same lanes per row, chunk order and sum tree), and the
    first linear matches the oracle."""
    lins, parts, xs, ys, xhost = _g32_pass("g32pass", chained=False)
    ref = [bqd.linear_w4a8_group32(wq, s16, None, x) for (_, wq, s16), x in zip(parts, xs)]
    p = bqd.DecodePass(lins, xs, ys)
    assert p.sources() == [-1] * len(lins)
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        p.run()
        sync()
        assert p.error_word() == 0
        for i, (y, yr) in enumerate(zip(ys, ref)):
            assert torch.equal(y, yr), (rep, i)
    _g32_oracle_first(parts, xhost, ys[0])


def test_decode_pass_group32_chained():
    """The same two group-32 layers chained through the exchange (fp32
    activations): every output equals the chain launched one linear at a
    time, over three passes; the first linear matches the oracle.  (Each
    group-32 output is a sum in fp32 whose rounding depends on the lanes'
    order, so further links are compared with the per-linear chain, which
    sums in the same order, not with an oracle chain.)"""
    lins, parts, xs, ys, xhost = _g32_pass("g32chain", chained=True)
    ref, xr = [], xs[0]
    for i, (W, wq, s16) in enumerate(parts):
        ref.append(bqd.linear_w4a8_group32(wq, s16, None, xr))
        xr = ref[-1][:parts[i + 1][0].shape[1]] if i + 1 < len(parts) else None
    p = bqd.DecodePass(lins, xs, ys)
    src = p.sources()
    assert src[0] == -1 and all(v >= 0 for v in src[1:])
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        p.run()
        sync()
        assert p.error_word() == 0
        for i, (y, yr) in enumerate(zip(ys, ref)):
            assert torch.equal(y, yr), (rep, i)
    _g32_oracle_first(parts, xhost, ys[0])


def test_decode_pass_rejects_descriptors_for_another_grid():
    """Descriptors encoded for another grid size are refused in the kernel
    (error bit 1, nothing computed) instead of being misread."""
    lins, xs, ys, parts = _pass_fixture(tag="passgrid")
    p = bqd.DecodePass(lins, xs, ys)
    grid = int(p.desc[4:8].cpu().view(torch.int32).item())
    bad = torch.tensor([grid + 1], dtype=torch.int32).view(torch.uint8).to(p.desc.device)
    good = p.desc[4:8].clone()
    for y in ys:
        y.fill_(float("nan"))
    p.desc[4:8] = bad
    p.run()
    sync()
    assert p.error_word() & 2
    assert all(torch.isnan(y).all() for y in ys)
    p.desc[4:8] = good
    p.clear_error()
    p.run()
    sync()
    assert p.error_word() == 0 and not any(torch.isnan(y).any() for y in ys)


@pytest.mark.parametrize("kind", ["rowwise", "group32"])
def test_decode_pass_instance_matches_the_encoded_step(kind):
    """The encoder picks 4 chunks per lane per step when every linear is
    group-32 and 8 otherwise; a launch of the other instance on those
    descriptors is refused in the kernel (error bit 1, nothing computed), and
    the encoded one then runs clean."""
    if kind == "rowwise":
        lins, xs, ys, _ = _pass_fixture(tag="passslots")
    else:
        lins, _, xs, ys, _ = _g32_pass("g32slots", chained=True)
    p = bqd.DecodePass(lins, xs, ys)
    want = 8 if kind == "rowwise" else 4
    assert p.slots == want
    assert int(p.desc[16:20].cpu().view(torch.int32).item()) == want  # the header's slots word
    for y in ys:
        y.fill_(float("nan"))
    p.slots = 12 - want
    p.run()
    sync()
    assert p.error_word() & 2
    assert all(torch.isnan(y).all() for y in ys)
    p.slots = want
    p.clear_error()
    p.run()
    sync()
    assert p.error_word() == 0 and not any(torch.isnan(y).any() for y in ys)


# ------------------------------------------------ packed 6-bit lm_head --
@pytest.mark.parametrize("N,K", [(3, 256), (37, 1536), (5, 4096)])
def test_quantize_weights_q6k_bit_exact(N, K):
    """Load-time 6-bit quantisation: ql, qh, sc and d bit-identical to the
    oracle's quantiser + packer (with a zero row, a zero sub-block and tiny
    sub-blocks under a large one)."""
    W = I.normal(f"gpu/q6k/{N}/{K}/W", (N, K), 0.02, device=DEV)
    W[0].zero_()
    if N > 1:
        W[1, 16:32] = 0.0
        W[1, 256 * (K // 512):] *= 1e-3
    w = bqd.quantize_weights_q6k(W)
    sync()
    q, sc, d = O.quantize_weights_q6k(npy(W))
    ql, qh = O.pack_q6k(q)
    assert np.array_equal(npy(w.ql), ql) and np.array_equal(npy(w.qh), qh)
    assert np.array_equal(npy(w.sc), sc) and np.array_equal(f16bits(w.d), d)


def _q6k_random(N, K, tag):
    """Every byte pattern of ql/qh (all codes), int8 scales over the whole
    int8 range, fp16 super-block scales."""
    ql = I.random_words(f"gpu/q6k/{tag}/ql", (N, K // 8), device=DEV).view(torch.uint8).view(N, K // 2)
    qh = I.random_words(f"gpu/q6k/{tag}/qh", (N, K // 16), device=DEV).view(torch.uint8).view(N, K // 4)
    sc = I.uniform_int(f"gpu/q6k/{tag}/sc", (N, K // 16), -128, 127, device=DEV, dtype=torch.int8)
    d = I.normal(f"gpu/q6k/{tag}/d", (N, K // 256), 1e-3, device=DEV, dtype=torch.float16)
    return bqd.Q6KWeights(ql, qh, sc, d)


@pytest.mark.parametrize("N,K", [(1, 256), (37, 768), (300, 1536), (2049, 1536)])
def test_gemv_q6k_matches_oracle(N, K):
    """In-register decode of the packed fields against the oracle, every
    (r, lanes) configuration; rows past a tile and chunks past a row."""
    w = _q6k_random(N, K, f"{N}/{K}")
    x16 = I.normal(f"gpu/q6k/{N}/{K}/x", K, 1.0, device=DEV, dtype=torch.float16)
    ql, qh, sc, d = npy(w.ql), npy(w.qh), npy(w.sc), f16bits(w.d)
    yr = O.gemv_q6k_f16(ql, qh, sc, d, f16bits(x16))
    q = O.unpack_q6k(ql, qh).astype(np.float64)
    e = (d.view(np.float16).astype(np.float64)[:, :, None] * sc.reshape(N, K // 256, 16)).reshape(N, K // 16)
    ax = np.abs(npy(x16).astype(np.float64))
    mag = (np.abs(e) * (np.abs(q) * ax).reshape(N, K // 16, 16).sum(2)).sum(1)
    for r, L in ((0, 0), (1, 16), (2, 32), (4, 64), (8, 16), (1, 64), (1, 8), (2, 8), (8, 8)):
        y = bqd.gemv_q6k_f16(w, x16, r=r, lanes_per_row=L)
        sync()
        assert rel_err(npy(y), yr, mag).max() <= TOL, (r, L)


def test_gemv_q6k_of_quantised_weights_tracks_the_int8_expansion():
    """Quantise W to the packed form on the GPU, expand the codes to int8
    with per-16 fp32 scales d*sc (the page's load-time expansion): the
    packed GEMV equals the float64 product of the expansion."""
    N, K = 512, 1536
    W = I.normal("gpu/q6k/exp/W", (N, K), 0.02, device=DEV)
    w = bqd.quantize_weights_q6k(W)
    x16 = I.normal("gpu/q6k/exp/x", K, 1.0, device=DEV, dtype=torch.float16)
    y = bqd.gemv_q6k_f16(w, x16)
    sync()
    q = O.unpack_q6k(npy(w.ql), npy(w.qh)).astype(np.float64)
    e = (npy(w.d).astype(np.float64)[:, :, None] * npy(w.sc).reshape(N, K // 256, 16)).reshape(N, K // 16)
    Wd = np.repeat(e, 16, axis=1) * q
    ref = Wd @ npy(x16).astype(np.float64)
    mag = np.abs(Wd) @ np.abs(npy(x16).astype(np.float64))
    assert rel_err(npy(y), ref, mag).max() <= TOL


# ------------------------------------------------------- INT8-X (3,5,8) --
def _int8x_codes(N, K, dist, tag):
    if dist == "page":
        return I.int8_codes_by_band(f"gpu/i8x/{tag}", (N, K))
    if dist == "bytes":
        return I.uniform_int(f"gpu/i8x/{tag}", (N, K), -128, 127, dtype=torch.int8)
    if dist == "l1":
        return I.uniform_int(f"gpu/i8x/{tag}", (N, K), -3, 3, dtype=torch.int8)
    return I.int8_codes_by_band(f"gpu/i8x/{tag}", (N, K), shares=(0, 0, 1000))


@pytest.mark.parametrize("dist", ["page", "bytes", "l1", "l3"])
@pytest.mark.parametrize("N,K", [(1, 512), (5, 1536), (37, 3584), (9, 18944)])
def test_gemv_int8x_matches_oracle(N, K, dist):
    """In-register INT8-X decode + W8A8 GEMV against the oracle (its own
    encoding and decoder): acc bit-exact, y within tolerance; every rows
    setting, rows past N included."""
    q = _int8x_codes(N, K, dist, f"{N}/{K}/{dist}")
    qx = I.uniform_int(f"gpu/i8x/{N}/{K}/x", K, -127, 127, device=DEV, dtype=torch.int8)
    sx = torch.tensor([0.0173], device=DEV)
    w = bqd.int8x_encode(q, 0.0042, device=DEV)
    acc_r, y_r = O.gemv_int8x(O.int8x_encode(q.numpy()), npy(qx), 0.0173, 0.0042)
    for rows in (0, 1, 2, 8):
        y, acc = bqd.gemv_int8x(w, qx, sx, acc=True, rows=rows)
        sync()
        assert np.array_equal(npy(acc), acc_r), rows
        mag = np.abs(y_r)
        assert np.all(np.abs(npy(y).astype(np.float64) - y_r) <= TOL * np.where(mag > 0, mag, 1.0)), rows


@pytest.mark.parametrize("N,K", [(3584, 3584), (4608, 3584), (17, 32), (8192, 8192), (1000, 1536), (33, 8224),
                                 (3584, 18944), (8192, 12800), (100, 24576)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_wide_workgroups_give_the_same_bits(N, K, dtype):
    """The automatic configuration runs few-row linears (K <= 24576: 1 to 12
    chunks per lane, 1 to 3 activation groups per thread) in 1024-thread
    workgroups (one wave per row): codes, scale, accumulators and y equal the
    256-thread kernel's bit for bit, for the fused linear and for the GEMV on
    a producer's codes."""
    w = I.random_words(f"gpu/wide/{N}/{K}/w", (N, K // 8), device=DEV)
    sw = I.normal(f"gpu/wide/{N}/{K}/s", N, 0.003, device=DEV).abs() + 1e-4
    b = I.normal(f"gpu/wide/{N}/{K}/b", N, 0.01, device=DEV)
    x = I.normal(f"gpu/wide/{K}/x", K, 1.0, device=DEV).to(dtype)
    y0, q0, s0, a0 = bqd.linear_w4a8(w, sw, b, x, want_q=True, want_acc=True)
    y1, q1, s1, a1 = bqd.linear_w4a8(w, sw, b, x, want_q=True, want_acc=True, r=1, lanes_per_row=32)
    g0, ga0 = bqd.gemv_w4a8(w, sw, b, q0, s0, acc=True)
    g1, ga1 = bqd.gemv_w4a8(w, sw, b, q0, s0, acc=True, r=1, lanes_per_row=16)
    sync()
    assert torch.equal(q0, q1) and torch.equal(s0, s1)
    assert torch.equal(a0, a1) and torch.equal(y0, y1)
    assert torch.equal(ga0, ga1) and torch.equal(g0, g1) and torch.equal(g0, y0)
