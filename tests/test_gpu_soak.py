"""Opt-in soak of the persistent pass's exchange: BQD_SOAK=<passes>.

Two chains as a decoder chains them, in one launch per pass, run BQD_SOAK
times each: the full Qwen2-7B-shaped stream (28 layers + lm_head, 113
per-row linears, the 8-chunk-step kernel instance) and the Gemma-shaped
one (35 layers, 140 group-32 linears, the 4-chunk-step instance).  Every
pass's outputs are compared bit for bit with the chain launched one linear
at a time, and its error word must stay 0; the test stops at the first
difference.  Between passes the outputs are poisoned with NaN, and
every few passes other work (a 64 MiB read-modify-write) changes what the
caches hold, so the passes do not all start from the same state."""
import os
import sys
import time

import pytest
import torch

import bit_quantized_decode_quantize_amd as bqd

pytestmark = pytest.mark.gpu
PASSES = int(os.environ.get("BQD_SOAK", "0") or 0)


def _soak(p, ref, tag):
    ref_bits = torch.cat(ref).view(torch.int32)
    bounds = torch.tensor([0] + [y.numel() for y in ref]).cumsum(0)
    noise = torch.zeros(16 << 20, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.time()
    for k in range(PASSES):
        for y in p.outputs:
            y.fill_(float("nan"))
        if k % 5 == 2:
            noise.add_(1)
        p.run()
        bits = torch.cat(p.outputs).view(torch.int32)
        bad = torch.nonzero(bits != ref_bits)
        err = p.error_word()
        assert err == 0, f"{tag} pass {k}: error word {err}"
        if bad.numel():
            j = int(bad[0, 0])
            lin = int(torch.searchsorted(bounds, j, right=True)) - 1
            pytest.fail(f"{tag} pass {k}: {bad.numel()} outputs differ, first in linear {lin} row "
                        f"{j - int(bounds[lin])}")
        if (k + 1) % 500 == 0 or k + 1 == PASSES:
            print(f"[soak] {tag}: {k + 1} passes bit-equal, {time.time() - t0:.1f} s", file=sys.stderr, flush=True)


@pytest.mark.skipif(PASSES <= 0, reason="opt-in: set BQD_SOAK to the number of passes")
def test_chained_stream_soak():
    from bit_quantized_decode_quantize_amd import decode_stream as DS
    s = DS.QwenW4A8Stream(layers=28, device="cuda", persistent=False)
    p = s.chained_pass()
    assert p.slots == 8
    ref, x = [], s.linears[0]["x"]
    for i, d in enumerate(s.linears):
        y = bqd.linear_w4a8(d["wq"], d["sw"], d["b"], x)
        ref.append(y)
        x = y[:s.linears[i + 1]["K"]] if i + 1 < len(s.linears) else None
    _soak(p, ref, "qwen")


@pytest.mark.skipif(PASSES <= 0, reason="opt-in: set BQD_SOAK to the number of passes")
def test_chained_group32_stream_soak():
    from bit_quantized_decode_quantize_amd import workloads as WL
    s = WL.GemmaG32Stream(device="cuda")
    p = s.make_pass(chained=True)
    assert p.slots == 4
    ref, x = [], p.inputs[0]
    for i, d in enumerate(s.linears):
        y = bqd.linear_w4a8_group32(d["wq"], d["s16"], None, x)
        ref.append(y)
        x = y[:s.linears[i + 1]["K"]] if i + 1 < len(s.linears) else None
    _soak(p, ref, "gemma")
