"""Host-side checks of the C ABI that need no GPU.

The library loads, exports every function include/bqd.h declares, and its
argument validation rejects bad calls before anything touches a device.
Every call here is built to fail validation (fake, non-null device pointers
never reach a kernel), so the tests are safe on a GPU machine too.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest
import torch

import bit_quantized_decode_quantize_amd as bqd
import oracle as O
from bit_quantized_decode_quantize_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULL, SHAPE, ALIGN, BOUND, DTYPE, CONFIG, LAUNCH, DEVICE = 0, -1, -2, -3, -4, -5, -6, -7, -8
P = 0x10000          # a fake, 64 KiB-aligned "device" address: never dereferenced
P4 = P + 4           # 4-byte but not 16-byte aligned


def header_functions():
    txt = open(os.path.join(ROOT, "include", "bqd.h"), encoding="utf-8").read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s+(\w+)\s*\(", txt, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) >= 16
    lib = bqd.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bqd.ENTRY_POINTS)


def test_version_and_status_strings():
    assert bqd.abi_version() == 4
    for s in (OK, NULL, SHAPE, ALIGN, BOUND, DTYPE, CONFIG, LAUNCH, DEVICE):
        assert bqd.status_string(s)
    assert bqd.status_string(12345) == "unknown status"


def test_init_reports_device_state():
    rc = bqd.lib().bqd_init()
    assert rc in (OK, DEVICE)
    if not torch.cuda.is_available():
        assert rc == DEVICE


L = None


def _lib():
    return bqd.lib()


@pytest.mark.parametrize("args,expected", [
    # (wq, sw, bias, qx, sx, y, acc, N, K, r, lanes)
    ((None, P, None, P, P, P, None, 8, 64, 0, 0), NULL),
    ((P, P, None, P, P, None, None, 8, 64, 0, 0), NULL),
    ((P, P, None, P, P, P, None, -1, 64, 0, 0), SHAPE),
    ((P, P, None, P, P, P, None, 8, 0, 0, 0), SHAPE),
    ((P, P, None, P, P, P, None, 8, 36, 0, 0), SHAPE),                # K % 8
    ((P, P, None, P, P, P, None, 8, 2113664 + 8, 0, 0), BOUND),      # past the int32 bound
    ((P4, P, None, P, P, P, None, 8, 64, 0, 0), ALIGN),
    ((P, P, None, P4, P, P, None, 8, 64, 0, 0), ALIGN),
    ((P, P + 2, None, P, P, P, None, 8, 64, 0, 0), ALIGN),
    ((P, P, P + 1, P, P, P, None, 8, 64, 0, 0), ALIGN),
    ((P, P, None, P, P, P, None, 8, 64, 3, 0), CONFIG),
    ((P, P, None, P, P, P, None, 8, 64, 4, 8), CONFIG),
    ((P, P, None, P, P, P, None, 8, 64, 16, 16), CONFIG),
])
def test_gemv_w4a8_validation(args, expected):
    assert _lib().gemv_w4a8(*args, None) == expected


def test_other_entry_points_validate_before_launch():
    L = _lib()
    # quantize_act(x, dtype, M, K, qx, sx, stream)
    assert L.quantize_act(P, 2, 1, 64, P, P, None) == DTYPE
    assert L.quantize_act(None, 0, 1, 64, P, P, None) == NULL
    assert L.quantize_act(P, 0, -1, 64, P, P, None) == SHAPE
    assert L.quantize_act(P4, 0, 1, 64, P, P, None) == ALIGN
    assert L.quantize_act(P, 0, 1, 44, P, P, None) == SHAPE
    assert L.quantize_act(P, 0, 1, 2113664 + 8, P, P, None) == BOUND
    # the general path: K % 8 == 0 up to the int32 bound for gemv_w4a8,
    # linear_w4a8, quantize_act and the automatic verify; other kernels keep K % 32
    assert L.linear_w4a8(P, P, None, P, 0, P, None, None, None, 8, 44, 0, 0, None) == SHAPE
    assert L.linear_w4a8(P, P, None, P, 0, P, None, None, None, 8, 2113664 + 8, 0, 0, None) == BOUND
    assert L.gemm_w4a8_verify(P, P, None, P, P, P, None, 2, 8, 44, 0, None, 0, None) == SHAPE
    assert L.gemm_w4a8_verify(P, P + 0x1000, None, P + 0x2000, P + 0x3000, P + 0x4000, None, 2, 8, 40, 3,
                              None, 0, None) == CONFIG                      # impl 1-3 need K % 32
    assert L.gemv_w4a8_group32(P, P, None, P, P, P, None, 8, 40, 0, 0, None) == SHAPE
    assert L.gemm_w4a8_verify_workspace_bytes(2, 8, 40) == 0
    # linear_w4a8(wq, sw, bias, x, dtype, y, qx_out, sx_out, acc, N, K, r, lanes, stream)
    assert L.linear_w4a8(P, P, None, P, 7, P, None, None, None, 8, 64, 0, 0, None) == DTYPE
    assert L.linear_w4a8(P, P, None, P4, 0, P, None, None, None, 8, 64, 0, 0, None) == ALIGN
    assert L.linear_w4a8(P, P, None, P, 0, P, P4, None, None, 8, 64, 0, 0, None) == ALIGN
    assert L.linear_w4a8(P, P, None, P, 0, P, None, None, None, 8, 64, 5, 0, None) == CONFIG
    # group-32
    assert L.gemv_w4a8_group32(P, P + 1, None, P, P, P, None, 8, 64, 0, 0, None) == ALIGN
    assert L.gemv_w4a8_group32(P, P, None, P, P, P, None, 8, 96 + 8, 0, 0, None) == SHAPE
    assert L.linear_w4a8_group32(P, None, None, P, 0, P, None, None, None, 8, 64, 0, 0, None) == NULL
    # W8A16: K above the LDS staging limit for fp16 activations
    assert L.gemv_w8a16_group32(P, P, P, P, 8, 65536, 0, 0, None) == BOUND
    assert L.gemv_w8a16_group32(P, P, P4, P, 8, 64, 0, 0, None) == ALIGN
    # verify: token count bound, impl
    assert L.gemm_w4a8_verify(P, P, None, P, P, P, None, 17, 8, 64, 0, None, 0, None) == BOUND
    assert L.gemm_w4a8_verify(P, P, None, P, P, P, None, 2, 8, 64, 9, None, 0, None) == CONFIG
    assert L.gemm_w4a8_verify(P, P, None, P, P, P, None, 2, 8, 64, 4, None, 0, None) == CONFIG
    assert L.gemm_w4a8_verify(P, P + 0x1000, None, P + 0x2000, P + 0x3000, P + 0x4000, None, 2, 8, 64, 3,
                              P + 0x5000 + 16, 1024, None) == ALIGN         # workspace not 256-byte aligned
    assert L.gemm_w4a8_verify(P, P + 0x1000, None, P + 0x2000, P + 0x3000, P + 0x4000, None, 2, 8, 64, 3,
                              P + 0x4000, 1024, None) == SHAPE             # workspace over y
    assert L.gemm_w4a8_verify_workspace_bytes(0, 8, 64) == 0
    assert L.gemm_w4a8_verify_workspace_bytes(2, 8, 40) == 0
    assert L.gemm_w4a8_verify(P, P, None, P, P, P, None, -1, 8, 64, 0, None, 0, None) == SHAPE
    # weight quantisers
    assert L.quantize_weights_int4_rowwise(P, 8, 36, P, P, None) == SHAPE
    assert L.quantize_weights_int4_group32(P4, 8, 64, P, P, None) == ALIGN
    assert L.quantize_weights_int8_group32(None, 8, 64, P, P, None) == NULL


def test_layer_forward_validates_every_linear_first():
    L = _lib()
    good = bqd.LinearW4A8(P, P + 0x1000, 0, 8, 64, 0, 0, 0)
    bad_k = bqd.LinearW4A8(P, P + 0x1000, 0, 8, 40, 0, 0, 0)
    bad_kind = bqd.LinearW4A8(P, P + 0x1000, 0, 8, 64, 3, 0, 0)
    xs = (C.c_void_p * 2)(P + 0x2000, P + 0x3000)
    ys = (C.c_void_p * 2)(P + 0x3000, P + 0x4000)
    arr = (bqd.LinearW4A8 * 2)(good, bad_k)
    assert L.layer_w4a8_forward(arr, 2, C.cast(xs, C.c_void_p), 0, C.cast(ys, C.c_void_p), None) == SHAPE
    arr = (bqd.LinearW4A8 * 2)(good, bad_kind)
    assert L.layer_w4a8_forward(arr, 2, C.cast(xs, C.c_void_p), 0, C.cast(ys, C.c_void_p), None) == DTYPE
    assert L.layer_w4a8_forward(arr, 65, C.cast(xs, C.c_void_p), 0, C.cast(ys, C.c_void_p), None) == SHAPE
    assert L.layer_w4a8_forward(None, 0, None, 0, None, None) == OK


def _no_device():
    return bqd.lib().bqd_init() == DEVICE


def test_outputs_may_not_overlap_what_the_launch_reads():
    """Every entry point refuses an output that overlaps one of its inputs
    or another output: workgroups read the inputs while others write."""
    L = _lib()
    N, K = 8, 64
    A = [P + 0x1000 * i for i in range(16)]   # disjoint 4 KiB windows
    wq, sw, bias, qx, sx, y, acc, x = A[:8]
    # gemv_w4a8(wq, sw, bias, qx, sx, y, acc, N, K, r, lanes, stream)
    g = L.gemv_w4a8
    assert g(wq, sw, bias, qx, sx, qx, None, N, K, 0, 0, None) == SHAPE       # y over qx
    assert g(wq, sw, bias, qx, sx, y, y + 16, N, K, 0, 0, None) == SHAPE      # acc over y
    assert g(wq, sw, bias, qx, sx, wq + 16, None, N, K, 0, 0, None) == SHAPE  # y inside the weights
    assert g(wq, sw, bias, qx, sx, sx, None, N, K, 0, 0, None) == SHAPE
    # linear_w4a8(wq, sw, bias, x, dtype, y, qx_out, sx_out, acc, N, K, r, lanes, stream)
    f = L.linear_w4a8
    assert f(wq, sw, bias, x, 0, x, None, None, None, N, K, 0, 0, None) == SHAPE           # y is x
    assert f(wq, sw, bias, x, 0, y, x + 128, None, None, N, K, 0, 0, None) == SHAPE       # qx_out in x
    assert f(wq, sw, bias, x, 1, y, None, x + 124, None, N, K, 0, 0, None) == SHAPE       # sx_out in fp16 x
    assert f(wq, sw, bias, x, 0, y, qx, y + 28, None, N, K, 0, 0, None) == SHAPE          # sx_out in y
    assert f(wq, sw, bias, x, 0, y, None, None, bias, N, K, 0, 0, None) == SHAPE          # acc over bias
    # group-32: s16 is [N, K/32] fp16, acc_g [N, K/32] int32
    h = L.gemv_w4a8_group32
    assert h(wq, sw, bias, qx, sx, y, sw + 16, N, K, 0, 0, None) == SHAPE                 # acc_g over s16
    assert h(wq, sw, bias, qx, sx, qx + 32, None, N, K, 0, 0, None) == SHAPE
    h = L.linear_w4a8_group32
    assert h(wq, sw, bias, x, 0, x + 252, None, None, None, N, K, 0, 0, None) == SHAPE
    assert h(wq, sw, bias, x, 0, y, y, None, None, N, K, 0, 0, None) == SHAPE            # qx_out over y
    # linear_rmsnorm_w4a8: every output apart from h, delta, gamma and each other
    r = L.linear_rmsnorm_w4a8
    hh, dd, gg, ho = A[8:12]
    assert r(wq, sw, bias, hh, dd, gg, 1e-6, ho, gg, None, None, None, N, K, 0, 0, None) == SHAPE   # y over gamma
    assert r(wq, sw, bias, hh, dd, gg, 1e-6, ho, y, ho + 64, None, None, N, K, 0, 0, None) == SHAPE  # qx_out in h_out
    assert r(wq, sw, bias, hh, dd, gg, 1e-6, ho, y, qx, dd, None, N, K, 0, 0, None) == SHAPE      # sx_out in delta
    assert r(wq, sw, bias, hh, dd, gg, 1e-6, ho, y, None, None, ho, N, K, 0, 0, None) == SHAPE    # acc over h_out
    # quantize_act, the producers, verify and the W8A16 head
    assert L.quantize_act(x, 0, 2, K, x + 256, sx, None) == SHAPE      # codes over token 1
    assert L.quantize_act(x, 0, 2, K, qx, x + 508, None) == SHAPE
    assert L.quantize_act(x, 0, 2, K, qx, qx + 64, None) == SHAPE     # sx over the codes of token 1
    rq = L.add_rmsnorm_quant
    assert rq(hh, dd, gg, 1e-6, hh + 16, None, qx, sx, 2, K, None) == SHAPE   # shifted h_out
    assert rq(hh, dd, gg, 1e-6, None, gg, qx, sx, 2, K, None) == SHAPE        # y_out over gamma
    assert rq(hh, dd, gg, 1e-6, ho, ho, qx, sx, 2, K, None) == SHAPE          # h_out and y_out one buffer
    assert rq(hh, dd, gg, 1e-6, None, None, hh, sx, 2, K, None) == SHAPE      # codes over h
    assert L.swiglu_quant(x, x + 256, qx, sx, 2, K, None) == SHAPE
    assert L.swiglu_quant(x, ho, ho + 16, sx, 2, K, None) == SHAPE
    assert L.gemm_w4a8_verify(wq, sw, bias, qx, sx, qx + 64, None, 2, N, K, 0, None, 0, None) == SHAPE  # y over token 1
    assert L.gemm_w4a8_verify(wq, sw, bias, qx, sx, y, y + 32, 2, N, K, 0, None, 0, None) == SHAPE
    assert L.gemv_w8a16_group32(wq, sw, x, x + 64, N, K, 0, 0, None) == SHAPE
    # a layer: y[i] may be x[i+1], never x[i] itself
    lin = bqd.LinearW4A8(wq, sw, 0, N, K, 0, 0, 0)
    arr = (bqd.LinearW4A8 * 2)(lin, lin)
    xs = (C.c_void_p * 2)(x, y)
    bad = (C.c_void_p * 2)(y, y)
    assert L.layer_w4a8_forward(arr, 2, C.cast(xs, C.c_void_p), 0, C.cast(bad, C.c_void_p), None) == SHAPE
    if _no_device():
        # the same calls with disjoint buffers pass every host check and reach
        # the device lookup (no device here)
        assert g(wq, sw, bias, qx, sx, y, acc, N, K, 0, 0, None) == DEVICE
        assert f(wq, sw, bias, x, 0, y, qx, sx, acc, N, K, 0, 0, None) == DEVICE
        assert r(wq, sw, bias, hh, dd, gg, 1e-6, ho, y, qx, sx, acc, N, K, 0, 0, None) == DEVICE
        assert rq(hh, dd, gg, 1e-6, hh, dd, qx, sx, 2, K, None) == DEVICE   # in place is allowed
        assert L.quantize_act(x, 0, 2, K, qx, sx, None) == DEVICE
        assert L.swiglu_quant(x, ho, qx, sx, 2, K, None) == DEVICE
        assert L.gemm_w4a8_verify(wq, sw, bias, qx, sx, y, acc, 2, N, K, 0, None, 0, None) == DEVICE
        assert L.gemv_w8a16_group32(wq, sw, x, y, N, K, 0, 0, None) == DEVICE
        good = (C.c_void_p * 2)(y, acc)
        assert L.layer_w4a8_forward(arr, 2, C.cast(xs, C.c_void_p), 0, C.cast(good, C.c_void_p), None) == DEVICE


def test_host_pack_helpers_match_oracle():
    q = I.uniform_int("abi/pack", (37, 96), -8, 7).to(torch.int8)
    q[0, :16] = torch.arange(-8, 8, dtype=torch.int8)
    w = bqd.pack_int4_rows_host(q)
    assert np.array_equal(w.numpy().view(np.uint32), O.pack_int4(q.numpy()))
    assert torch.equal(bqd.unpack_int4_rows_host(w), q)
    words = I.random_words("abi/words", (11, 12))
    assert np.array_equal(bqd.unpack_int4_rows_host(words).numpy(),
                          O.unpack_int4(words.numpy().view(np.uint32)))
    bad = q.clone()
    bad[3, 3] = 9
    with pytest.raises(bqd.BQDError):
        bqd.pack_int4_rows_host(bad)


def test_binding_rejects_mismatched_buffers_before_the_call():
    """Shape checks live in the binding: the C ABI cannot see buffer sizes."""
    with pytest.raises((ValueError, TypeError)):
        bqd.bqd._dev(torch.zeros(4), "x", (torch.float32,))   # CPU tensor


def test_decode_pass_encode_validates_and_serialises():
    L = _lib()
    n = 2
    nbytes = L.decode_pass_desc_bytes(n)
    assert nbytes == 32 + 2 * 96
    host = (C.c_uint8 * nbytes)()
    mk = C.c_int32(0)
    sb = C.c_size_t(0)
    sl = C.c_int32(0)
    # clear of the weights (a: P .. P + 0x2BC00), x[1]: 18944 fp32 = 0x12800 bytes
    X0, X1, Y0, Y1 = P + 0x400000, P + 0x410000, P + 0x440000, P + 0x450000

    def enc(lins, nbytes=nbytes, n=n, dt=0, x=(X0, X1), y=(Y0, Y1)):
        arr = (bqd.LinearW4A8 * len(lins))(*lins)
        xs = (C.c_void_p * 2)(*x)
        ys = (C.c_void_p * 2)(*y)
        return L.decode_pass_encode(arr, n, C.cast(xs, C.c_void_p), dt, C.cast(ys, C.c_void_p),
                                    C.cast(host, C.c_void_p), nbytes, C.byref(mk), C.byref(sb), C.byref(sl))

    a = bqd.LinearW4A8(P, P + 0x400, 0, 100, 3584, 0, 0, 0)
    b = bqd.LinearW4A8(P + 0x1000, P + 0x500, P + 0x600, 7, 18944, 0, 0, 0)
    assert enc([a, b], nbytes=100) == SHAPE
    assert enc([a, b], dt=4) == DTYPE
    assert enc([a, bqd.LinearW4A8(P, P, 0, 7, 64, 2, 0, 0)]) == DTYPE       # unknown scale kind
    assert enc([a, bqd.LinearW4A8(P, P, 0, 7, 96, 1, 0, 0)]) == SHAPE       # group-32: K % 256
    assert enc([a, bqd.LinearW4A8(P, P + 8, 0, 7, 256, 1, 0, 0)]) == ALIGN  # group-32 scales: 16-byte aligned
    assert enc([a, bqd.LinearW4A8(P, P, 0, 7, 64, 0, 2, 16)]) == CONFIG     # the pass picks the split
    assert enc([a, bqd.LinearW4A8(P, P, 0, 0, 64, 0, 0, 0)]) == SHAPE       # N = 0
    assert enc([a, bqd.LinearW4A8(P4, P, 0, 7, 64, 0, 0, 0)]) == ALIGN
    assert enc([a, bqd.LinearW4A8(P, P, 0, 7, 40, 0, 0, 0)]) == SHAPE       # K % 32
    assert enc([a, bqd.LinearW4A8(P, P, 0, 7, bqd.BQD_MAX_PASS_K + 32, 0, 0, 0)]) == BOUND  # LDS
    assert enc([a, b], n=0) == SHAPE
    # a linear whose output overlaps its own activation: its workgroups would
    # write y while others still read x (fp32 x[1] spans 4 * 18944 bytes, fp16 half that)
    assert enc([a, b], y=(Y0, X1 + 4 * 18944 - 4)) == SHAPE
    assert enc([a, b], y=(Y0, X1 - 4 * 7 + 4)) == SHAPE
    assert enc([a, b], y=(X0 + 4 * 3584 - 4, Y1)) == SHAPE
    assert enc([a, b], y=(Y0, X1 + 2 * 18944 - 4), dt=1) == SHAPE
    # an activation read before the launch that a later linear overwrites:
    # workgroups run ahead, so it could be overwritten before every reader
    # has it (x[0] over y[1])
    assert enc([a, b], y=(Y0, X0 + 64)) == SHAPE
    # outputs overlapping each other (each is written once per pass)
    assert enc([a, b], y=(Y0, Y0 + 4 * 100 - 4)) == SHAPE
    valid = DEVICE if not torch.cuda.is_available() else OK   # encoding needs the device's grid
    assert enc([a, b], y=(Y0, Y0 + 4 * 100)) == valid
    # x[1] inside y[0] is the chain (read from the exchange): fp32 only, and
    # wholly inside.  y[0] of 20000 rows holds x[1] (18944 values) 16 values in.
    Y1b = P + 0x480000
    wide = bqd.LinearW4A8(P + 0x10000000, P + 0x400, 0, 20000, 3584, 0, 0, 0)
    chained = dict(x=(X0, Y0 + 64), y=(Y0, Y1b))
    assert enc([wide, b], **chained) == valid
    assert enc([wide, b], x=(X0, Y0 + 4 * 20000 - 64), y=(Y0, Y1b)) == SHAPE     # runs past y[0]'s end
    assert enc([wide, b], dt=1, x=(X0, Y0 + 64), y=(Y0, Y1b)) == DTYPE          # fp16 over an fp32 output
    # an output over a linear's weights, scales or bias (read, and prefetched
    # before the activation is ready, through the caches)
    W, S, B = P + 0x100000, P + 0x200000, P + 0x300000
    c = bqd.LinearW4A8(W, S, B, 64, 64, 0, 0, 0)                      # 2048 weight bytes, 256 scale bytes
    assert enc([a, c], y=(W + 2048 - 4, Y1)) == SHAPE
    assert enc([a, c], y=(Y0, S + 252)) == SHAPE
    assert enc([a, c], y=(B - 4 * 64 + 4, Y1)) == SHAPE
    assert enc([a, c], y=(W + 2048, Y1)) != SHAPE
    rc = enc([a, b])
    if not torch.cuda.is_available():
        assert rc == DEVICE
        return
    assert rc == OK and mk.value == 18944
    import struct
    raw = bytes(host)
    hn, grid, hk, words = struct.unpack("<4i", raw[:16])
    assert (hn, hk, words) == (2, 18944, 0) and 0 < grid <= 1024   # nothing read from the exchange
    assert sb.value == (64 + 1024 * 16) * 4                        # err line + epoch lines
    f = struct.unpack("<5Q14i", raw[16 + 96:16 + 192])
    assert f[:5] == (P + 0x1000, P + 0x500, P + 0x600, X1, Y1)
    N, C_, base, extra, lshift, r, iters, batches, steps, xin, xout, xdt, kind, _ = f[5:]
    assert (N, C_, base, extra, xin, xout, xdt, kind) == (7, 592, 7 // grid, 7 % grid, -1, -1, 1, 0)
    assert lshift in (4, 5, 6) and r in (1, 2)
    assert iters == -(-592 // (1 << lshift)) and steps == -(-iters * r // 8)
    # the chain: y[0] gets 20000 exchange words (+ its offset mod 16 bytes),
    # x[1] starts 16 words into them
    assert enc([wide, b], **chained) == OK
    raw = bytes(host)
    words = struct.unpack("<4i", raw[:16])[3]
    xin0, xout0 = struct.unpack("<2i", raw[16 + 76:16 + 84])
    xin1, xout1 = struct.unpack("<2i", raw[16 + 96 + 76:16 + 96 + 84])
    assert (xin0, xout0, xout1) == (-1, (Y0 >> 2) & 3, -1) and xin1 == xout0 + 16
    assert words == -(-(20000 + 3) // 64) * 64 and sb.value == (64 + 1024 * 16 + 2 * words) * 4


def test_decode_pass_launch_validates_before_launch():
    L = _lib()
    WS = (64 + 1024 * 16) * 4                # the smallest workspace: no exchange
    assert L.decode_pass_w4a8(P, 0, 64, 8, P, WS, 0, None) == SHAPE
    assert L.decode_pass_w4a8(None, 2, 64, 8, P, WS, 0, None) == NULL
    assert L.decode_pass_w4a8(P, 2, 64, 8, None, WS, 0, None) == NULL
    assert L.decode_pass_w4a8(P, 2, 40, 8, P, WS, 0, None) == SHAPE
    assert L.decode_pass_w4a8(P, 2, 64, 8, P, WS, -1, None) == CONFIG
    assert L.decode_pass_w4a8(P + 8, 2, 64, 8, P, WS, 0, None) == ALIGN
    assert L.decode_pass_w4a8(P, 2, 64, 8, P + 64, WS, 0, None) == ALIGN   # the workspace is 256-byte aligned
    assert L.decode_pass_w4a8(P, 2, 64, 8, P, WS - 256, 0, None) == SHAPE  # smaller than any workspace
    assert L.decode_pass_w4a8(P, 2, 64, 8, P, WS + 4, 0, None) == SHAPE    # not a workspace size
    assert L.decode_pass_w4a8(P, 2, 64, 6, P, WS, 0, None) == CONFIG            # slots: 4 or 8


def test_read_probe_validates_before_launch():
    L = _lib()
    # read_probe(buf, bytes, sink, grid, unroll, stream)
    assert L.read_probe(P, 40, P, 8, 1, None) == SHAPE
    assert L.read_probe(P, 64, P, 0, 1, None) == SHAPE
    assert L.read_probe(P, 64, P, 8, 3, None) == CONFIG
    assert L.read_probe(None, 64, P, 8, 1, None) == NULL
    assert L.read_probe(P + 8, 64, P, 8, 1, None) == ALIGN
    assert L.read_probe(P, 0, None, 8, 1, None) == OK


def test_gemv_w4a16_validates_before_launch():
    L = _lib()
    # gemv_w4a16(wq, sw, bias, x16, y, N, K, r, lanes, stream)
    assert L.gemv_w4a16(P, P, None, P, P, 8, 48, 0, 0, None) == SHAPE
    assert L.gemv_w4a16(P, P, None, P, P, 8, 65536, 0, 0, None) == BOUND
    assert L.gemv_w4a16(P, P, None, None, P, 8, 64, 0, 0, None) == NULL
    assert L.gemv_w4a16(P, P, None, P + 8, P, 8, 64, 0, 0, None) == ALIGN
    assert L.gemv_w4a16(P, P, None, P, P, 8, 64, 3, 0, None) == CONFIG
    assert L.gemv_w4a16(P, P, None, P, P, 0, 64, 0, 0, None) == OK


def test_producers_validate_before_launch():
    L = _lib()
    # add_rmsnorm_quant(h, delta, gamma, eps, h_out, y_out, qx, sx, M, K, stream)
    assert L.add_rmsnorm_quant(P, None, P, 1e-6, None, None, P, P, 2, 48, None) == SHAPE
    assert L.add_rmsnorm_quant(P, None, P, 1e-6, None, None, P, P, 2, 32800, None) == BOUND
    assert L.add_rmsnorm_quant(P, None, P, -1.0, None, None, P, P, 2, 64, None) == SHAPE
    assert L.add_rmsnorm_quant(P, None, P, float("inf"), None, None, P, P, 2, 64, None) == SHAPE
    assert L.add_rmsnorm_quant(P, None, P, float("nan"), None, None, P, P, 2, 64, None) == SHAPE
    assert L.add_rmsnorm_quant(P, None, P, 1e-6, None, None, P, P, -1, 64, None) == SHAPE
    assert L.add_rmsnorm_quant(None, None, P, 1e-6, None, None, P, P, 2, 64, None) == NULL
    assert L.add_rmsnorm_quant(P, None, None, 1e-6, None, None, P, P, 2, 64, None) == NULL
    assert L.add_rmsnorm_quant(P, None, P, 1e-6, None, None, P, None, 2, 64, None) == NULL
    assert L.add_rmsnorm_quant(P, P4, P, 1e-6, None, None, P, P, 2, 64, None) == ALIGN
    assert L.add_rmsnorm_quant(P, None, P, 1e-6, None, P + 8, P, P, 2, 64, None) == ALIGN
    assert L.add_rmsnorm_quant(P, None, P, 1e-6, None, None, P, P, 0, 64, None) == OK
    # swiglu_quant(gu, h_out, qx, sx, M, I, stream)
    assert L.swiglu_quant(P, None, P, P, 2, 40, None) == SHAPE
    assert L.swiglu_quant(P, None, P, P, 2, 32800, None) == BOUND
    assert L.swiglu_quant(None, None, P, P, 2, 64, None) == NULL
    assert L.swiglu_quant(P, None, P, None, 2, 64, None) == NULL
    assert L.swiglu_quant(P, None, P, P, 2, 64, None) == NULL  # h_out is required
    assert L.swiglu_quant(P, P4, P, P, 2, 64, None) == ALIGN
    assert L.swiglu_quant(P, None, P, P, 0, 64, None) == OK


def test_q6k_entry_points_validate_before_launch():
    L = _lib()
    # quantize_weights_q6k(W, N, K, ql, qh, sc, d, stream)
    assert L.quantize_weights_q6k(P, 4, 128, P, P, P, P, None) == SHAPE
    assert L.quantize_weights_q6k(P, 4, 65536 + 256, P, P, P, P, None) == BOUND
    assert L.quantize_weights_q6k(P, -1, 256, P, P, P, P, None) == SHAPE
    assert L.quantize_weights_q6k(P, 4, 256, P, None, P, P, None) == NULL
    assert L.quantize_weights_q6k(P4, 4, 256, P, P, P, P, None) == ALIGN
    assert L.quantize_weights_q6k(P, 4, 256, P4, P, P, P, None) == ALIGN
    assert L.quantize_weights_q6k(P, 0, 256, None, None, None, None, None) == OK
    # gemv_q6k_f16(ql, qh, sc, d, x16, y, N, K, r, lanes, stream)
    assert L.gemv_q6k_f16(P, P, P, P, P, P, 4, 96, 0, 0, None) == SHAPE
    assert L.gemv_q6k_f16(P, P, P, P, P, P, 4, 65536, 0, 0, None) == BOUND
    assert L.gemv_q6k_f16(P, P, None, P, P, P, 4, 256, 0, 0, None) == NULL
    assert L.gemv_q6k_f16(P, P4, P, P, P, P, 4, 256, 0, 0, None) == ALIGN
    assert L.gemv_q6k_f16(P, P + 8, P, P, P, P, 4, 256, 0, 0, None) == ALIGN
    assert L.gemv_q6k_f16(P, P, P, P, P, P, 4, 256, 0, 4, None) == CONFIG
    assert L.gemv_q6k_f16(P, P, P, P, P + 8, P, 4, 256, 0, 0, None) == ALIGN
    assert L.gemv_q6k_f16(P, P, P, P, P, P, 4, 256, 3, 0, None) == CONFIG
    assert L.gemv_q6k_f16(P, P, P, P, P, P, 0, 256, 0, 0, None) == OK


def _lib_int8x_encode(q):
    """The library's host encoder into numpy arrays of its stated sizes."""
    L = _lib()
    q = np.ascontiguousarray(q, np.int8)
    n = q.size
    counts = (C.c_int64 * 3)()
    assert L.int8x_counts_host(q.ctypes.data, n, counts) == OK
    sizes = (C.c_int64 * 7)()
    assert L.int8x_stream_bytes_host(n, counts, sizes) == OK
    names = ("b1", "b2", "l1", "l2", "l3", "b1_blk", "b2_blk")
    arr = {k: np.full(sz // (1 if k == "l3" else 4), 0x5A, np.uint8 if k == "l3" else np.uint32)
           for k, sz in zip(names, sizes)}
    assert L.int8x_encode_host(q.ctypes.data, n, *[arr[k].ctypes.data for k in names]) == OK
    return arr, tuple(counts)


@pytest.mark.parametrize("shape,dist", [((1, 512), "laplace"), ((7, 1536), "bytes"), ((3, 3584), "laplace"),
                                        ((2, 512), "l3"), ((1, 1024), "l1")])
def test_int8x_host_encoder_matches_the_oracle(shape, dist):
    """The library's encoder (its own code) writes the oracle's streams bit
    for bit; the padding words are zero."""
    rng = np.random.default_rng(31)
    if dist == "laplace":
        q = np.clip(np.round(rng.laplace(0, 4.3, shape)), -127, 127).astype(np.int8)
    elif dist == "bytes":
        q = rng.integers(-128, 128, shape, dtype=np.int8)
    elif dist == "l3":
        q = rng.choice(np.int8([-128, -16, 16, 127]), shape)
    else:
        q = rng.integers(-3, 4, shape, dtype=np.int8)
    arr, counts = _lib_int8x_encode(q)
    e = O.int8x_encode(q)
    assert counts == (e["n1"], e["n2"], e["n3"])
    n1, n2, n3 = counts
    used = {"b1": (q.size + 31) // 32, "b2": (n2 + n3 + 31) // 32, "l1": (3 * n1 + 31) // 32,
            "l2": (5 * n2 + 31) // 32, "l3": n3, "b1_blk": len(e["b1_blk"]), "b2_blk": len(e["b2_blk"])}
    for k, m in used.items():
        assert np.array_equal(arr[k][:m], e[k][:m]), k
        assert len(arr[k]) >= m
        if k not in ("b1_blk", "b2_blk"):
            assert not arr[k][m:].any(), k  # padding zeroed


def test_int8x_entry_points_validate():
    L = _lib()
    counts = (C.c_int64 * 3)(5, 3, 2)
    sizes = (C.c_int64 * 7)()
    assert L.int8x_stream_bytes_host(10, counts, sizes) == OK
    assert list(sizes) == [16, 16, 16, 16, 16, 8, 8]
    assert L.int8x_stream_bytes_host(11, counts, sizes) == SHAPE
    assert L.int8x_counts_host(None, 4, counts) == NULL
    assert L.int8x_counts_host(P, 0, counts) == SHAPE
    sz = (C.c_int64 * 7)(64, 16, 16, 16, 16, 8, 8)
    huge = (C.c_int64 * 7)(64, 16, (1 << 28) + 16, 16, 16, 8, 8)
    # gemv_int8x(b1, b2, l1, l2, l3, b1_blk, b2_blk, sizes, qx, sx, sw, y, acc, N, K, rows, stream)
    args = [P] * 7
    assert L.gemv_int8x(*args, sz, P, P, 1.0, P, None, 1, 500, 0, None) == SHAPE
    assert L.gemv_int8x(*args, sz, P, P, 1.0, P, None, 1, 66048, 0, None) == BOUND
    assert L.gemv_int8x(*args, None, P, P, 1.0, P, None, 1, 512, 0, None) == NULL
    assert L.gemv_int8x(*args, sz, P, None, 1.0, P, None, 1, 512, 0, None) == NULL
    assert L.gemv_int8x(*args, sz, P4, P, 1.0, P, None, 1, 512, 0, None) == ALIGN
    assert L.gemv_int8x(*args, sz, P, P, 1.0, P, None, 1, 512, 3, None) == CONFIG
    small = (C.c_int64 * 7)(4, 16, 16, 16, 16, 8, 8)  # b1 shorter than N*K bits
    assert L.gemv_int8x(*args, small, P, P, 1.0, P, None, 1, 512, 0, None) == SHAPE
    short_blk = (C.c_int64 * 7)(64, 16, 16, 16, 16, 4, 8)  # block sums need N*K/512 + 1 entries
    assert L.gemv_int8x(*args, short_blk, P, P, 1.0, P, None, 1, 512, 0, None) == SHAPE
    assert L.gemv_int8x(*args, huge, P, P, 1.0, P, None, 1, 512, 0, None) == BOUND
    assert L.gemv_int8x(*args, sz, P, P, 1.0, P, None, 0, 512, 0, None) == OK


def test_linear_rmsnorm_validates_before_launch():
    L = _lib()
    # linear_rmsnorm_w4a8(wq, sw, bias, h, delta, gamma, eps, h_out, y, qx, sx, acc, N, K, r, lanes, stream)
    f = L.linear_rmsnorm_w4a8
    assert f(P, P, None, P, None, P, 1e-6, None, P, None, None, None, 4, 48, 0, 0, None) == SHAPE
    assert f(P, P, None, P, None, P, 1e-6, None, P, None, None, None, 4, 8224, 0, 0, None) == BOUND
    assert f(P, P, None, P, None, P, -1.0, None, P, None, None, None, 4, 64, 0, 0, None) == SHAPE
    assert f(P, P, None, P, None, P, 1e-6, P + 128, P, None, None, None, 4, 64, 0, 0, None) == SHAPE  # h_out overlaps h
    assert f(P, P, None, P, P + 4096, P, 1e-6, P + 4096 + 64, P, None, None, None, 4, 64, 0, 0, None) == SHAPE
    assert f(P, P, None, None, None, P, 1e-6, None, P, None, None, None, 4, 64, 0, 0, None) == NULL
    assert f(P, P, None, P, None, None, 1e-6, None, P, None, None, None, 4, 64, 0, 0, None) == NULL
    assert f(P, P, None, P + 8, None, P, 1e-6, None, P, None, None, None, 4, 64, 0, 0, None) == ALIGN
    assert f(P, P, None, P, None, P, 1e-6, None, P, None, None, None, 4, 64, 3, 0, None) == CONFIG
    assert f(P, P, None, P, None, P, 1e-6, None, P, None, None, None, 0, 64, 0, 0, None) == OK


def test_bench_reads_the_pass_kernel_code_hash():
    """bench.py keys the committed HBM-traffic figure to the sha256 of
    k_decode_pass's machine code in the library's gfx950 code object: the
    reader finds it in the in-tree build, and the committed summary holds
    both of its fields."""
    import bench
    sha = bench.kernel_code_sha256(bqd.bqd.LIB_PATH)
    assert sha is not None and re.fullmatch(r"[0-9a-f]{64}", sha)
    assert bench.kernel_code_sha256(bqd.bqd.LIB_PATH, needle="no_such_kernel") is None
    assert bench.kernel_code_sha256(os.path.join(ROOT, "no_such_library.so")) is None
    for path in bench.TRAFFIC.values():
        if not os.path.exists(path):
            continue
        text = open(path).read()
        assert re.search(r"^traffic_bytes_per_launch: \d+$", text, re.M), path
        assert re.search(r"^kernel_code_sha256: [0-9a-f]{64}$", text, re.M), path
        sym = re.search(r"^kernel_symbol: (\S+)$", text, re.M)
        assert sym, path
        # the symbol exists in the in-tree build (its code may have changed since)
        assert bench.kernel_code_sha256(bqd.bqd.LIB_PATH, sym.group(1), exact=True) is not None, path


def test_binding_constants_match_the_header():
    """Every BQD_ constant the binding defines has the value include/bqd.h
    gives it, and the status codes these tests use are the header's."""
    text = open(os.path.join(ROOT, "include", "bqd.h")).read()
    defs = {m.group(1): int(m.group(2)) for m in re.finditer(r"^#define (BQD_\w+) \(?(-?\d+)\)?", text, re.M)}
    mod = bqd.bqd
    shared = [n for n in defs if hasattr(mod, n)]
    assert {"BQD_MAX_K", "BQD_MAX_K_ANY", "BQD_MAX_TOKENS", "BQD_MAX_PROD_K", "BQD_MAX_PASS_K", "BQD_INT8X_BLOCK", "BQD_F32",
            "BQD_F16", "BQD_SCALE_ROW_F32", "BQD_SCALE_GROUP32_F16"} <= set(shared)
    for n in shared:
        assert getattr(mod, n) == defs[n], n
    codes = {"BQD_OK": OK, "BQD_ERR_NULL": NULL, "BQD_ERR_SHAPE": SHAPE, "BQD_ERR_ALIGN": ALIGN,
             "BQD_ERR_BOUND": BOUND, "BQD_ERR_DTYPE": DTYPE, "BQD_ERR_CONFIG": CONFIG, "BQD_ERR_LAUNCH": LAUNCH,
             "BQD_ERR_DEVICE": DEVICE}
    for n, v in codes.items():
        assert defs[n] == v, n


def test_bench_refuses_more_than_one_gpu():
    """bench.py --gpus N > 1 exits with status 2 and a message, before any
    GPU work."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""


def test_bench_inputs_digest_names_the_data():
    """The digest bench.py puts on each line changes with any input byte and
    not with the order of equal calls."""
    import bench
    a = torch.arange(64, dtype=torch.float32)
    b = torch.ones(8, dtype=torch.int8)
    d = bench.inputs_digest(a, b)
    assert re.fullmatch(r"[0-9a-f]{16}", d)
    assert bench.inputs_digest(a, b) == d
    a2 = a.clone()
    a2[5] += 1
    assert bench.inputs_digest(a2, b) != d
    assert bench.inputs_digest(b, a) != d
    assert bench.inputs_digest(a, None, b) == d
