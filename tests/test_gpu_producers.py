"""GPU parity of the activation producers fused with the quantisation
(residual add + RMSNorm + quant, SwiGLU + quant) against the CPU oracle,
through the C ABI.

The producers' fp32 values come from fixed sequences of IEEE operations, so
every comparison here is bit-exact: the int8 codes, the scale s^x and the
fp32 values (h + delta, y, h).  Inputs are seeded on the device and handed
to the oracle as they are; nothing the oracle sees comes from the GPU path.
"""
import numpy as np
import pytest
import torch

import oracle as O
from bit_quantized_decode_quantize_amd import bqd
from bit_quantized_decode_quantize_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda"


def npy(t):
    return t.detach().cpu().numpy()


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def sync():
    torch.cuda.synchronize()


def _rms_inputs(M, K, tag, residual=True):
    h = I.normal(f"gpu/rms/{tag}/h", (M, K), 1.0, device=DEV)
    d = I.normal(f"gpu/rms/{tag}/d", (M, K), 0.5, device=DEV) if residual else None
    gamma = 1.0 + I.normal(f"gpu/rms/{tag}/g", K, 0.1, device=DEV)
    return h, d, gamma


def _check_rms(h, d, gamma, eps, M, K):
    h_out = torch.full((M, K), float("nan"), device=DEV)
    y_out = torch.full((M, K), float("nan"), device=DEV)
    qx, sx = bqd.add_rmsnorm_quant(h, gamma, eps, delta=d, h_out=h_out, y_out=y_out)
    sync()
    q, s, h1, y = O.add_rmsnorm_quant(npy(h), None if d is None else npy(d), npy(gamma), eps)
    assert np.array_equal(bits(npy(h_out)), bits(h1))
    assert np.array_equal(bits(npy(y_out)), bits(y))
    assert np.array_equal(bits(npy(sx)), bits(s))
    assert np.array_equal(npy(qx), q)


@pytest.mark.parametrize("residual", [True, False])
@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (2, 3584), (1, 18944), (5, 1536), (1, 32768)])
def test_add_rmsnorm_quant_bit_exact(M, K, residual):
    """Codes, s^x, h + delta and y bit-identical to the oracle; K from one
    32-block to the 32768 maximum (up to 8 values per thread, ragged against
    the 1024 threads)."""
    h, d, gamma = _rms_inputs(M, K, f"{M}/{K}", residual)
    _check_rms(h, d, gamma, 1e-6, M, K)


def test_add_rmsnorm_quant_special_tokens():
    """eps = 0 with a zero token (codes 0, s = 0), a constant token (codes
    +-127), a one-spike token, a token with 1 % of its values x20, and a
    token scaled by 2^40 in one batch."""
    K = 3584
    h, _, gamma = _rms_inputs(5, K, "special", residual=False)
    h[0].zero_()
    h[1].fill_(-0.375)
    h[2].zero_()
    h[2, 17] = 3.0
    idx = I.distinct_indices("gpu/rms/special/outliers", K, K // 100).to(DEV)
    h[3, idx] *= 20.0
    h[4] *= 2.0 ** 40
    for eps in (0.0, 1e-6):
        _check_rms(h, None, gamma, eps, 5, K)
    qx, sx = bqd.add_rmsnorm_quant(h, gamma, 0.0)
    sync()
    assert npy(sx)[0] == 0.0 and not npy(qx)[0].any()
    assert np.all(npy(qx)[1] < 0)  # a negative constant normalises to -1, times gamma > 0


def test_add_rmsnorm_quant_in_place_residual():
    """h_out may be h itself: the residual stream is updated in place."""
    M, K = 2, 3584
    h, d, gamma = _rms_inputs(M, K, "inplace")
    h0 = npy(h).copy()
    qx, sx = bqd.add_rmsnorm_quant(h, gamma, 1e-6, delta=d, h_out=h)
    sync()
    q, s, h1, _ = O.add_rmsnorm_quant(h0, npy(d), npy(gamma), 1e-6)
    assert np.array_equal(bits(npy(h)), bits(h1))
    assert np.array_equal(npy(qx), q) and np.array_equal(bits(npy(sx)), bits(s))


def test_add_rmsnorm_without_quantisation_writes_the_values_only():
    M, K = 2, 1536
    h, d, gamma = _rms_inputs(M, K, "noq")
    y_out = torch.empty(M, K, device=DEV)
    assert bqd.add_rmsnorm_quant(h, gamma, 1e-6, delta=d, y_out=y_out, quantize=False) == (None, None)
    sync()
    _, _, _, y = O.add_rmsnorm_quant(npy(h), npy(d), npy(gamma), 1e-6)
    assert np.array_equal(bits(npy(y_out)), bits(y))


def _gu(M, I_, tag, gate_sigma=2.0):
    g = I.normal(f"gpu/swiglu/{tag}/g", (M, I_), gate_sigma, device=DEV)
    u = I.normal(f"gpu/swiglu/{tag}/u", (M, I_), 1.0, device=DEV)
    return torch.cat([g, u], dim=1).contiguous()


def _check_swiglu(gu, M, I_):
    h_out = torch.full((M, I_), float("nan"), device=DEV)
    qx, sx = bqd.swiglu_quant(gu, h_out=h_out)
    sync()
    q, s, h = O.swiglu_quant(npy(gu))
    assert np.array_equal(bits(npy(h_out)), bits(h))
    assert np.array_equal(bits(npy(sx)), bits(s))
    assert np.array_equal(npy(qx), q)


@pytest.mark.parametrize("M,I_", [(1, 32), (3, 96), (1, 18944), (4, 6144), (1, 32768)])
def test_swiglu_quant_bit_exact(M, I_):
    """h = silu(g) * u, codes and s^x bit-identical to the oracle."""
    _check_swiglu(_gu(M, I_, f"{M}/{I_}"), M, I_)


def test_swiglu_quant_extreme_gates():
    """Gates across the exponential's clamp and overflow: +-30, +-88, +-89,
    +-104, +-1e4, 0, +-1e-30, denormal-range products; then an all-zero gate
    (s = 0, every code 0)."""
    I_ = 1024
    gu = _gu(2, I_, "extreme")
    special = torch.tensor([30.0, -30.0, 88.0, -88.0, 89.0, -89.0, 104.0, -104.0, 1e4, -1e4, 0.0,
                            1e-30, -1e-30, 87.3, -87.3, 103.0], device=DEV)
    gu[0, :special.numel()] = special
    gu[0, I_:I_ + 4] = torch.tensor([1e-38, -1e-38, 3e38, -3e38], device=DEV) * 1e-3
    _check_swiglu(gu, 2, I_)
    gu[1, :I_] = 0.0
    qx, sx = bqd.swiglu_quant(gu)
    sync()
    assert npy(sx)[1] == 0.0 and not npy(qx)[1].any()


def test_swiglu_without_quantisation_writes_h_only():
    gu = _gu(1, 6144, "noq")
    h_out = torch.empty(1, 6144, device=DEV)
    assert bqd.swiglu_quant(gu, h_out=h_out, quantize=False) == (None, None)
    sync()
    assert np.array_equal(bits(npy(h_out)), bits(O.swiglu_quant(npy(gu))[2]))


def test_producer_then_gemv_equals_consumer_fused_linear():
    """RMSNorm+quant then the int8 GEMV, against RMSNorm (fp32 out) then the
    linear that quantises in its prologue: the same codes, so the same y
    bits; SwiGLU likewise for the down projection."""
    K, N, I_ = 3584, 4608, 18944
    h, d, gamma = _rms_inputs(1, K, "chain")
    W = I.normal("gpu/chain/W", (N, K), 0.02, device=DEV)
    wq, sw = bqd.quantize_weights_int4_rowwise(W)
    b = I.normal("gpu/chain/b", N, 0.01, device=DEV)
    qx, sx = bqd.add_rmsnorm_quant(h, gamma, 1e-6, delta=d)
    y1 = bqd.gemv_w4a8(wq, sw, b, qx.view(K), sx)
    yv = torch.empty(1, K, device=DEV)
    bqd.add_rmsnorm_quant(h, gamma, 1e-6, delta=d, y_out=yv, quantize=False)
    y2 = bqd.linear_w4a8(wq, sw, b, yv.view(K))
    Wd = I.normal("gpu/chain/Wd", (K, I_), 0.02, device=DEV)
    wqd, swd = bqd.quantize_weights_int4_rowwise(Wd)
    gu = _gu(1, I_, "chain")
    qd, sd = bqd.swiglu_quant(gu)
    z1 = bqd.gemv_w4a8(wqd, swd, None, qd.view(I_), sd)
    hv = torch.empty(1, I_, device=DEV)
    bqd.swiglu_quant(gu, h_out=hv, quantize=False)
    z2 = bqd.linear_w4a8(wqd, swd, None, hv.view(I_))
    sync()
    assert torch.equal(y1, y2) and torch.equal(z1, z2)
    # and against the oracle: its own producer's codes feed its GEMV
    q, s, _, _ = O.add_rmsnorm_quant(npy(h), npy(d), npy(gamma), 1e-6)
    wr, sr = O.prepare_int4_rowwise(npy(W))
    acc, yr = O.gemv_w4a8(wr, sr, npy(b), q[0], float(s[0]))
    err = O.rel_err_rowwise(npy(y1), yr, sr, s[0], acc, npy(b))
    assert err.max() <= 1e-5


def test_producers_in_a_graph_replay_match_eager():
    """The two producers and their GEMVs captured in one HIP graph, replayed
    four times with eager work in between: every replay equals the eager
    result bit for bit."""
    K, I_ = 3584, 18944
    h, d, gamma = _rms_inputs(1, K, "graph")
    gu = _gu(1, I_, "graph")
    W = I.normal("gpu/graph/W", (2 * I_, K), 0.02, device=DEV)
    wq, sw = bqd.quantize_weights_int4_rowwise(W)
    qx = torch.empty(1, K, dtype=torch.int8, device=DEV)
    sx = torch.empty(1, device=DEV)
    qd = torch.empty(1, I_, dtype=torch.int8, device=DEV)
    sd = torch.empty(1, device=DEV)
    ygu = torch.empty(2 * I_, device=DEV)
    h1 = torch.empty(1, K, device=DEV)

    def step():
        bqd.add_rmsnorm_quant(h, gamma, 1e-6, delta=d, h_out=h1, qx=qx, sx=sx)
        bqd.gemv_w4a8(wq, sw, None, qx.view(K), sx, y=ygu)
        bqd.swiglu_quant(ygu.view(1, -1), qx=qd, sx=sd)

    step()
    sync()
    ref = [t.clone() for t in (qx, sx, ygu, qd, sd, h1)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        for t in (qx, sx, ygu, qd, sd, h1):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        sync()
        for a, r in zip((qx, sx, ygu, qd, sd, h1), ref):
            assert torch.equal(a, r)


@pytest.mark.parametrize("residual", [True, False])
@pytest.mark.parametrize("N,K", [(1, 32), (37, 1536), (4608, 3584), (300, 8192)])
def test_linear_rmsnorm_w4a8_matches_producer_and_oracle(N, K, residual):
    """RMSNorm + quantisation in the linear's prologue: the codes, s^x and
    h + delta of the oracle's add_rmsnorm_quant bit for bit, the oracle's
    accumulators, and the same y bits as add_rmsnorm_quant + gemv_w4a8."""
    h, d, gamma = _rms_inputs(1, K, f"lin/{N}/{K}", residual)
    h, d = h.view(K), (None if d is None else d.view(K))
    W = I.normal(f"gpu/linrms/{N}/{K}/W", (N, K), 0.02, device=DEV)
    wq, sw = bqd.quantize_weights_int4_rowwise(W)
    b = I.normal(f"gpu/linrms/{N}/{K}/b", N, 0.01, device=DEV)
    h_out = torch.full((K,), float("nan"), device=DEV)
    y, qx, sx, acc = bqd.linear_rmsnorm_w4a8(wq, sw, b, h, gamma, 1e-6, delta=d, h_out=h_out, want_q=True,
                                            want_acc=True)
    q2, s2 = bqd.add_rmsnorm_quant(h.view(1, K), gamma, 1e-6, delta=None if d is None else d.view(1, K))
    y2 = bqd.gemv_w4a8(wq, sw, b, q2.view(K), s2)
    sync()
    q, s, h1, _ = O.add_rmsnorm_quant(npy(h), None if d is None else npy(d), npy(gamma), 1e-6)
    assert np.array_equal(npy(qx), q) and np.array_equal(bits(npy(sx)).ravel(), bits(np.atleast_1d(s)))
    assert np.array_equal(bits(npy(h_out)), bits(h1))
    accr, yr = O.gemv_w4a8(O.pack_int4(O.unpack_int4(npy(wq).view(np.uint32))), npy(sw), npy(b), q, float(s))
    assert np.array_equal(npy(acc), accr)
    assert O.rel_err_rowwise(npy(y), yr, npy(sw), float(s), accr, npy(b)).max() <= 1e-5
    assert torch.equal(y, y2)
