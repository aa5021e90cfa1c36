"""The allocation-free entry point decode_pass_w4a8_static against the
ordinary one (decode_pass_w4a8) through the C ABI: two calls in a row, the
second with a smaller pass, each bit-equal to the ordinary entry point, and
the host-side bound on the workspace size."""
import ctypes as C

import pytest
import torch

import bit_quantized_decode_quantize_amd as bqd
from bit_quantized_decode_quantize_amd import inputs as I

DEV = torch.device("cuda:0")
pytestmark = pytest.mark.gpu


def _chained(tag, shapes):
    lins, ys = [], []
    for i, (N, K) in enumerate(shapes):
        wq, sw = bqd.quantize_weights_int4_rowwise(I.normal(f"gpu/{tag}/{i}/W", (N, K), 0.02, device=DEV))
        b = I.normal(f"gpu/{tag}/{i}/b", N, 0.01, device=DEV) if i % 2 == 0 else None
        lins.append(bqd.make_linear(wq, sw, b))
        ys.append(torch.full((N,), float("nan"), device=DEV))
    x0 = I.normal(f"gpu/{tag}/x", shapes[0][1], 1.0, device=DEV)
    xs = [x0] + [ys[i - 1][:K] for i, (_, K) in enumerate(shapes) if i > 0]
    return bqd.DecodePass(lins, xs, ys), ys


def _run_both(p, ys, err):
    """Ordinary entry point, then the static one into fresh outputs."""
    p.run()
    torch.cuda.synchronize()
    assert p.error_word() == 0
    ref = [y.clone() for y in ys]
    for y in ys:
        y.fill_(float("nan"))
    err.fill_(-1)
    p.run_static(err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for i, (y, r) in enumerate(zip(ys, ref)):
        assert torch.equal(y, r), i


def test_static_pass_equals_the_ordinary_entry_point_twice():
    torch.cuda.set_device(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    big = [(4608, 3584), (3584, 3584), (37888, 3584), (3584, 18944), (4608, 3584), (2048, 3584)]
    p1, ys1 = _chained("static/big", big)
    assert p1.sync_bytes <= bqd.BQD_STATIC_PASS_BYTES
    _run_both(p1, ys1, err)
    # a second, smaller pass with other descriptors over the same static
    # array (which still holds the first call's exchange words)
    small = [(1024, 512), (512, 1024), (256, 512)]
    p2, ys2 = _chained("static/small", small)
    assert p2.sync_bytes < p1.sync_bytes
    _run_both(p2, ys2, err)
    # and the first again, twice in a row (the array's state carries over)
    for _ in range(2):
        _run_both(p1, ys1, err)


def test_static_pass_refuses_a_workspace_beyond_its_array():
    torch.cuda.set_device(DEV)
    p, _ = _chained("static/bound", [(512, 256), (256, 512)])
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    L = bqd.lib()
    too_big = bqd.BQD_STATIC_PASS_BYTES + 256
    assert L.decode_pass_w4a8_static(p.desc.data_ptr(), p.n, p.max_k, p.slots, too_big, 0, err.data_ptr(), None) == -4
    assert L.decode_pass_w4a8_static(p.desc.data_ptr(), p.n, p.max_k, p.slots, p.sync_bytes, 0, None, None) == -1


def test_static_pass_replays_from_a_hip_graph():
    """The case the entry point is for: captured once into a HIP graph
    (nothing allocated inside the capture, the workspace cleared by a kernel)
    and replayed three times, with eager work between the replays; every
    replay's outputs equal the ordinary entry point's, bit for bit."""
    torch.cuda.set_device(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    p, ys = _chained("static/graph", [(4608, 3584), (3584, 3584), (8192, 3584), (3584, 8192)])
    p.run()
    torch.cuda.synchronize()
    assert p.error_word() == 0
    ref = [y.clone() for y in ys]
    p.run_static(err)  # warm: library set-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        p.run_static(err)
    other, other_ys = _chained("static/graph-other", [(1024, 512), (512, 1024)])
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        err.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0, rep
        for i, (y, r) in enumerate(zip(ys, ref)):
            assert torch.equal(y, r), (rep, i)
        other.run_static(err)  # eager use of the same static array between replays
        torch.cuda.synchronize()
        assert int(err.item()) == 0
