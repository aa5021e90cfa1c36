"""GPU parity of the benchmark workloads at their full sizes, in the launch
configurations bench.py times (rotation pools, per-linear HIP graphs, the
persistent pass), against the CPU oracle on sampled rows.

The oracle's inputs are regenerated from the same seeded streams on the
device the workload drew them on (so every value is the same) and
quantised by the oracle itself: no expected value comes from the GPU path.
"""
import numpy as np
import pytest
import torch

import oracle as O
import parity_log as P
from bit_quantized_decode_quantize_amd import inputs as I
from bit_quantized_decode_quantize_amd import workloads as WL
from bit_quantized_decode_quantize_amd import decode_stream as DS
from bit_quantized_decode_quantize_amd import bqd

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-5


def npy(t):
    return t.detach().cpu().numpy()


def f16bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _rows(N, name, count=96):
    idx = I.distinct_indices(f"gpu/wl/{name}/rows", N, min(count, N)).numpy()
    return np.unique(np.concatenate([idx, [0, N - 1]]))


def _check_rowwise_rows(y, W_rows, b_rows, x, rows):
    """Oracle on the sampled rows only: prepare, quantise x, GEMV."""
    wr, sr = O.prepare_int4_rowwise(W_rows)
    qxr, sxr = O.quantize_act(x)
    accr, yr = O.gemv_w4a8(wr, sr, b_rows, qxr, float(sxr))
    P.check_rowwise("", y[rows], yr, sr, sxr, accr, b_rows, TOL)


def _graph_replay(step, n):
    """Capture n consecutive steps in a HIP graph and replay it once."""
    step()  # warm (library init outside the capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            step()
    g.replay()
    torch.cuda.synchronize()


def test_single_gemv_pool_graph_replay():
    """The single Q-projection linear, one graph replay over the whole pool
    (every copy writes the one output): y matches the oracle."""
    w = WL.SingleGemvPool(device=DEV)
    w.y.fill_(float("nan"))
    _graph_replay(w.step, w.copies)
    y = npy(w.y)
    d = I.single_gemv_inputs(0, DEV)
    rows = _rows(w.N, "single")
    _check_rowwise_rows(y, npy(d["W"])[rows], npy(d["b"])[rows], npy(d["x"]), rows)


@pytest.mark.parametrize("persistent", [True, False])
def test_layer_pool(persistent):
    """One layer's four fused linears over the rotation pool.  Per-linear
    graph replay: every copy gives the same bits, matching the oracle on
    sampled rows.  Persistent: one launch chains every copy's linears as a
    decoder does (each reads the previous output), equal bit for bit to the
    same chain launched one linear at a time; its first linear reads the
    layer's own activation and matches the oracle on sampled rows."""
    w = WL.LayerPool(device=DEV, persistent=persistent)
    lins = I.qwen_layer_linears()
    if persistent:
        w.step()
        torch.cuda.synchronize()
        assert w.pass_.error_word() == 0
        flat = [e for lin in w.layers for e in lin]
        xr = flat[0]["x"]
        for i, e in enumerate(flat):
            yr = bqd.linear_w4a8(e["wq"], e["sw"], e["b"], xr)
            assert torch.equal(e["y"], yr), i
            xr = yr[:flat[i + 1]["K"]] if i + 1 < len(flat) else None
        checked = lins[:1]
    else:
        _graph_replay(w.step, w.copies)
        for k in range(len(lins)):
            y0 = w.layers[0][k]["y"]
            for c in range(1, w.copies):
                assert torch.equal(w.layers[c][k]["y"], y0)
        checked = lins
    for k, (name, N, K) in enumerate(checked):
        y0 = w.layers[0][k]["y"]
        rows = _rows(N, f"layer/{name}")
        W = DS.linear_weight_fp32("qwen/L0", name, 0, DEV)[torch.as_tensor(rows, device=DEV)]
        b = DS.layer_biases("qwen/L0", 0, DEV)[name]
        x = DS.layer_inputs("qwen/L0", 0, DEV)[name]
        _check_rowwise_rows(npy(y0), npy(W), npy(b)[rows], npy(x), rows)


def test_gemma_stream_layer_and_lm_head():
    """Two Gemma-shaped group-32 layers (fp16 x) and the W8A16 lm_head
    [262144, 1536], one graph replay of the token step, against the oracle
    on sampled rows."""
    w = WL.GemmaG32Stream(layers=2, device=DEV)
    _graph_replay(w.step, 1)
    for d in w.linears:
        rows = _rows(d["N"], f"gemma/{d['layer']}/{d['name']}", 64)
        W = I.normal(f"gemma/L{d['layer']}/{d['name']}/W", (d["N"], d["K"]), 0.02, 0, DEV)
        wr, s16r = O.prepare_int4_group32(npy(W)[rows])
        qxr, sxr = O.quantize_act(npy(d["x"]))
        accg, yr = O.gemv_w4a8_group32(wr, s16r, None, qxr, float(sxr))
        sg = s16r.view(np.float16).astype(np.float64)
        mag = float(sxr) * np.abs(sg * accg).sum(1)
        err = np.abs(npy(d["y"])[rows].astype(np.float64) - yr) / np.where(mag > 0, mag, 1.0)
        assert err.max() <= TOL, (d["name"], err.max())
    N, K = w.head_NK
    rows = _rows(N, "gemma/lm_head", 256)
    W = I.normal("gemma/lm_head/W", (N, K), 0.02, 0, DEV)[torch.as_tensor(rows, device=DEV)]
    q, s = O.quantize_weights_int8_group32(npy(W))
    yr = O.gemv_w8a16_group32(q, s, f16bits(w.head_x))
    sg = s.view(np.float16).astype(np.float64)
    ax = np.abs(f16bits(w.head_x).view(np.float16).astype(np.float64))
    mag = (sg * (np.abs(q).astype(np.float64).reshape(len(rows), -1, 32) * ax.reshape(-1, 32)).sum(2)).sum(1)
    err = np.abs(npy(w.head_y)[rows].astype(np.float64) - yr) / mag
    assert err.max() <= TOL, err.max()


@pytest.mark.parametrize("N,K", [(18944, 3584), (3584, 18944)])
@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_verify_pool(N, K, M):
    """The verify GEMM at its benchmark shapes, automatic kernel choice,
    graph replay over the pool: codes bit-exact, y of every token within
    tolerance of the oracle on sampled rows."""
    w = WL.VerifyPool(N, K, M, device=DEV)
    _graph_replay(w.step, w.copies)
    y = npy(w.y)
    rows = _rows(N, f"verify/{N}/{K}", 64)
    W = I.normal(f"verify/{N}x{K}/W", (N, K), 0.02, 0, DEV)[torch.as_tensor(rows, device=DEV)]
    wr, sr = O.prepare_int4_rowwise(npy(W))
    b = npy(I.normal(f"verify/{N}x{K}/b", N, 0.01, 0, DEV))[rows]
    qxr, sxr = O.quantize_act(npy(I.normal(f"verify/{N}x{K}/X", (M, K), 1.0, 0, DEV)))
    assert np.array_equal(npy(w.qx), qxr)
    accr, yr = O.gemm_w4a8_verify(wr, sr, b, qxr, sxr)
    for m in range(M):
        P.check_rowwise(f"token {m}", y[m][rows], yr[m], sr, sxr[m], accr[m], b, TOL)


@pytest.mark.parametrize("unroll", [1, 4, 8])
def test_read_probe_reads_every_word(unroll):
    """The read-ceiling kernel: workgroup b's sink word is the XOR of the
    16-byte words threads 0 and 1 of b read in the grid-stride loop."""
    from bit_quantized_decode_quantize_amd import bqd
    grid, n16 = 8, 8 * 256 * 5 + 37
    words = I.random_words("gpu/read_probe", n16 * 4, device=DEV)
    sink = torch.zeros(grid, dtype=torch.int32, device=DEV)
    bqd.read_probe(words, sink, grid, unroll)
    w = npy(words).view(np.uint32).reshape(n16, 4)
    fold = w[:, 0] ^ w[:, 1] ^ w[:, 2] ^ w[:, 3]
    stride = grid * 256
    expect = []
    for b in range(grid):
        a = np.uint32(0)
        for t in (0, 1):
            for i in range(b * 256 + t, n16, stride):
                a ^= fold[i]
        expect.append(a)
    assert np.array_equal(npy(sink).view(np.uint32), np.array(expect, np.uint32))


def test_decode_chain_modes_agree_and_match_the_oracle():
    """Two Qwen-shaped layers and the lm_head wired as a decoder, one graph
    replay per token as bench.py times it: RMSNorm in the consuming linear's
    prologue, producers writing int8 codes, and fp32 producers with linears
    that quantise in their prologue give identical bits everywhere; the first
    producer's codes and the first QKV output match the oracle."""
    s = DS.QwenW4A8Stream(layers=2, device=DEV, persistent=False)
    c = DS.DecodeChain(s)
    _graph_replay(lambda: c.step("prologue"), 1)
    ref = [d["y"].clone() for d in s.linears]
    for mode in ("producers", "fp32"):
        _graph_replay(lambda: c.step(mode), 1)
        for d, y in zip(s.linears, ref):
            assert torch.equal(d["y"], y), (mode, d["name"])
    # the first producer and the first QKV against the oracle
    q, sx, _, _ = O.add_rmsnorm_quant(npy(c.h_in), None, npy(c.gamma[0]), DS.RMS_EPS)
    qkv = c.by_layer[0]["qkv"]
    rows = _rows(qkv["N"], "chain/qkv")
    W = s.fp32_rows(qkv, torch.as_tensor(rows))
    wr, sr = O.prepare_int4_rowwise(npy(W))
    b = npy(qkv["b"])[rows]
    accr, yr = O.gemv_w4a8(wr, sr, b, q[0], float(sx[0]))
    P.check_rowwise("", npy(ref[0])[rows], yr, sr, sx[0], accr, b, TOL)
    qg, _ = bqd.add_rmsnorm_quant(c.h_in, c.gamma[0], DS.RMS_EPS)
    torch.cuda.synchronize()
    assert np.array_equal(npy(qg), q)


def test_gemma_packed_6bit_lm_head():
    """The Gemma token step with the packed 6-bit lm_head [262144, 1536], one
    graph replay: on sampled rows the packed fields equal the oracle's
    quantiser + packer and y matches the oracle's GEMV."""
    w = WL.GemmaG32Stream(layers=1, device=DEV, head="q6k")
    _graph_replay(w.step, 1)
    N, K = w.head_NK
    rows = _rows(N, "gemma/q6k", 256)
    W = I.normal("gemma/lm_head/W", (N, K), 0.02, 0, DEV)[torch.as_tensor(rows, device=DEV)]
    q, sc, d = O.quantize_weights_q6k(npy(W))
    ql, qh = O.pack_q6k(q)
    g = w.q6k
    assert np.array_equal(npy(g.ql)[rows], ql) and np.array_equal(npy(g.qh)[rows], qh)
    assert np.array_equal(npy(g.sc)[rows], sc) and np.array_equal(f16bits(g.d)[rows], d)
    x = f16bits(w.head_x)
    yr = O.gemv_q6k_f16(ql, qh, sc, d, x)
    e = (d.view(np.float16).astype(np.float64)[:, :, None] * sc.reshape(len(rows), K // 256, 16)).reshape(len(rows), -1)
    ax = np.abs(x.view(np.float16).astype(np.float64))
    mag = (np.abs(e) * (np.abs(q.astype(np.float64)) * ax).reshape(len(rows), K // 16, 16).sum(2)).sum(1)
    err = np.abs(npy(w.head_y)[rows].astype(np.float64) - yr) / mag
    assert err.max() <= TOL, err.max()


def test_int8x_pool_down_shape_matches_oracle():
    """INT8-X weights [3584, 18944] with the page's level shares, graph
    replay over the pool as bench.py times it: acc bit-exact on sampled rows
    against the oracle's own encoding and decoder."""
    w = WL.Int8XPool(3584, 18944, device=DEV)
    _graph_replay(w.step, w.copies)
    y = npy(w.y)
    q = I.int8_codes_by_band("int8x/3584x18944/q", (3584, 18944)).numpy()
    e = O.int8x_encode(q)
    rows = _rows(3584, "int8x")
    qx = npy(w.qx)
    for j in rows:
        row = O.int8x_decode(e, int(j) * 18944, 18944)
        acc = int(row.astype(np.int64) @ qx.astype(np.int64))
        ref = float(np.float32(0.0042)) * float(np.float32(0.0173)) * acc
        assert abs(float(y[j]) - ref) <= TOL * max(abs(ref), 1e-30), j
    acc_all = bqd.gemv_int8x(w.pool[0], w.qx, w.sx, acc=True)[1]
    torch.cuda.synchronize()
    assert np.array_equal(npy(acc_all)[rows], (q[rows].astype(np.int64) @ qx.astype(np.int64)).astype(np.int32))
