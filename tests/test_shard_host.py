"""Host-side checks of the tensor-parallel split (no GPU): the row shares
partition every fused linear, and, on the oracle, the two facts the split
rests on: int32 partial accumulators over K slices add up to the whole
accumulator, and the largest slice s^x is the whole activation's s^x."""
import numpy as np
import torch

import oracle as O
from bit_quantized_decode_quantize_amd import inputs as I
from bit_quantized_decode_quantize_amd import workloads as WL
from bit_quantized_decode_quantize_amd.decode_stream import _qwen_part_shapes


def test_row_shares_partition_each_fused_linear():
    for name in ("qkv", "gate_up"):
        parts, _ = _qwen_part_shapes()[name]
        N = sum(n for _, n in parts)
        for G in (1, 2, 4, 8):
            shares = [WL.shard_row_index(name, r, G, "cpu") for r in range(G)]
            allr = torch.cat(shares)
            assert allr.numel() == N and torch.equal(allr.sort().values, torch.arange(N))
            # each share holds the same slice of every part (whole heads, matching gate and up rows)
            for r, s in enumerate(shares):
                off = 0
                for _, n in parts:
                    inside = s[(s >= off) & (s < off + n)] - off
                    assert torch.equal(inside, torch.arange(r * n // G, (r + 1) * n // G))
                    off += n


def _case(N, K, seed):
    W = I.normal(f"host/shard/{seed}/W", (N, K), 0.02, seed, "cpu").numpy()
    x = I.normal(f"host/shard/{seed}/x", (K,), 1.0, seed, "cpu").numpy()
    return W, x


def test_oracle_k_slice_partials_sum_to_the_whole_accumulator():
    N, K, G = 96, 1024, 8
    W, x = _case(N, K, 3)
    wq, sw = O.prepare_int4_rowwise(W)
    qx, sx = O.quantize_act(x)
    acc, _ = O.gemv_w4a8(wq, sw, None, qx, float(sx))
    ks = K // G
    total = np.zeros(N, np.int64)
    for r in range(G):
        a, _ = O.gemv_w4a8(wq[:, r * ks // 8:(r + 1) * ks // 8].copy(), sw, None, qx[r * ks:(r + 1) * ks].copy(),
                           float(sx))
        total += a
    np.testing.assert_array_equal(total, acc.astype(np.int64))


def test_oracle_slice_scales_max_is_the_whole_scale():
    for K, G in ((3584, 8), (18944, 8), (1024, 4)):
        _, x = _case(4, K, K)
        x[K // 3] = 40.0  # the maximum inside one slice
        _, sx = O.quantize_act(x)
        ks = K // G
        s = [O.quantize_act(x[r * ks:(r + 1) * ks].copy())[1] for r in range(G)]
        assert np.float32(max(s)).view(np.uint32) == np.float32(sx).view(np.uint32)
