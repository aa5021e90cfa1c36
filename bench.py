"""Decode-stream benchmark: one step = one token's pass over the Qwen2-7B-shaped
28-layer W4A8 weight stream plus the int4 lm_head, all resident in HBM.

Each of the 113 linears (28 layers x {fused QKV, O, fused gate/up, down} +
lm_head) is one launch of the library's fused kernel: per-token activation
quantisation in the prologue, INT4 x INT8 dot products, int32 accumulation,
fp32 epilogue.  Prints one JSON line (rank 0, N=1).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for W4A8 decode GEMV; implied 28-layer tok/s"
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--layers", type=int, default=28)
    p.add_argument("--r", type=int, default=0, help="rows per lane group (0 = automatic)")
    p.add_argument("--lanes", type=int, default=0, help="lanes per row (0 = automatic)")
    p.add_argument("--per-linear", action="store_true",
                   help="one launch per linear instead of one persistent launch per step")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="before the timed region, run one plain device copy of this many MiB "
                        "(the reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    return p.parse_args()


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_decode_pass_qwen2-7b-28L_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "bit_quantized_decode_quantize_amd", "csrc", "bqd_kernels.hip")


def measured_traffic():
    """HBM bytes per pass launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (copy-calibrated), or None once the kernel source
    differs from the one the counters were taken on."""
    try:
        text = open(TRAFFIC_SUMMARY, encoding="utf-8").read()
        sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    vals = dict(re.findall(r"^(traffic_bytes_per_launch|kernel_source_sha256): (\S+)$", text, re.M))
    if vals.get("kernel_source_sha256") != sha or "traffic_bytes_per_launch" not in vals:
        return None
    return int(vals["traffic_bytes_per_launch"])


def cpu_baseline(stream, seconds):
    """The C oracle, single-threaded on this host, over layer 0 of the same
    stream (its four linears: activation quantisation + GEMV), repeated for
    about ``seconds``; reported as algorithmic GB/s and implied tok/s."""
    import numpy as np
    import oracle as O
    from bit_quantized_decode_quantize_amd import decode_stream as DS

    work = []
    for d in stream.linears[:4]:
        rows = __import__("torch").arange(d["N"])
        W = stream.fp32_rows(d, rows).cpu().numpy()
        w, s = O.prepare_int4_rowwise(W)
        del W
        b = None if d["b"] is None else d["b"].cpu().numpy()
        work.append((w, s, b, d["x"].cpu().numpy(), DS.algorithmic_bytes_linear(d["N"], d["K"], b is not None)))
    sample_bytes = sum(wk[4] for wk in work)
    reps, t0 = 0, time.perf_counter()
    while True:
        for w, s, b, x, _ in work:
            O.linear_w4a8(w, s, b, x)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gbs = sample_bytes * reps / el / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0 of the stream (fused QKV, O, gate/up, down: {sample_bytes} algorithmic bytes), "
                      f"{reps} passes in {el:.1f} s, single-threaded C; implied tok/s over the full "
                      f"stream {gbs * 1e9 / stream.bytes_per_step():.4f}"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {a.gpus} requested); the path's sharding "
              "is described in DESIGN.md", file=sys.stderr)
        sys.exit(2)
    import torch
    from bit_quantized_decode_quantize_amd import bqd
    from bit_quantized_decode_quantize_amd import decode_stream as DS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    s = DS.QwenW4A8Stream(layers=a.layers, device=dev, r=a.r, lanes_per_row=a.lanes,
                          persistent=not a.per_linear)
    print(f"[bench] stream built: {len(s.linears)} linears, {s.weight_bytes() / 1e9:.3f} GB packed, "
          f"{time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    st = torch.cuda.current_stream()
    if a.copy_calibration:
        src = torch.empty(a.copy_calibration << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy: {src.numel() * 4} bytes read, {dst.numel() * 4} bytes written",
              file=sys.stderr, flush=True)
        del src, dst

    for _ in range(a.warmup):
        s.step()
    torch.cuda.synchronize()

    # Timed region: K whole steps back to back on one stream.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(a.steps):
        s.step()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    step_bytes = s.bytes_per_step()
    gbs = step_bytes / (ms * 1e-3) / 1e9

    if s.persistent:
        # One launch per step: the pass kernel carries every byte.  Second
        # pass of the same K steps with events around each launch.
        evs = []
        for _ in range(a.steps):
            b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            b0.record(st)
            s.step()
            b1.record(st)
            evs.append((b0, b1))
        torch.cuda.synchronize()
        err = s.pass_.error_word()
        if err:
            raise RuntimeError(f"decode pass reported a wait time-out (error word {err})")
        dur_us = [b0.elapsed_time(b1) * 1e3 for b0, b1 in evs]
        avg_us = sum(dur_us) / len(dur_us)
        avg_bytes = step_bytes
        kernel = "k_decode_pass (persistent: whole token pass, 113 linears, one launch)"
    else:
        # Dominant kernel: the gate/up linears + lm_head (most of the bytes).
        # Second pass of the same K steps, each such launch bracketed by events.
        dom = [i for i, d in enumerate(s.linears) if d["name"] in ("gate_up", "lm_head")]
        evs = []
        for _ in range(a.steps):
            for i, d in enumerate(s.linears):
                if i in dom:
                    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    b0.record(st)
                    bqd.linear_w4a8(d["wq"], d["sw"], d["b"], d["x"], y=d["y"], r=a.r, lanes_per_row=a.lanes)
                    b1.record(st)
                    evs.append((b0, b1, i))
                else:
                    bqd.linear_w4a8(d["wq"], d["sw"], d["b"], d["x"], y=d["y"], r=a.r, lanes_per_row=a.lanes)
        torch.cuda.synchronize()
        dur_us = [b0.elapsed_time(b1) * 1e3 for b0, b1, _ in evs]
        dom_bytes = [DS.algorithmic_bytes_linear(s.linears[i]["N"], s.linears[i]["K"], s.linears[i]["b"] is not None)
                     for _, _, i in evs]
        avg_us = sum(dur_us) / len(dur_us)
        avg_bytes = sum(dom_bytes) / len(dom_bytes)
        kernel = "k_gemv_w4a8 (fused gate/up linears and lm_head, one launch per linear)"
    achieved = avg_bytes / (avg_us * 1e-6) / 1e9

    out = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": "qwen2-7b-shaped 28-layer W4A8 decode weight stream + int4 lm_head "
                               "(per-row scales, fused QKV and gate/up, fused act-quant)",
                   "launch": "per-linear" if a.per_linear else "persistent pass",
                   "layers": a.layers, "hidden": 3584, "kv_dim": 512, "intermediate": 18944,
                   "vocab": 152064, "global_batch": 1, "parallelism": "none",
                   "bytes_per_step": step_bytes, "packed_weight_bytes": s.weight_bytes()},
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tok_per_s": round(1e3 / ms, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if s.persistent else None,
                     "kernel": kernel,
                     "avg_launch_us": round(avg_us, 3), "avg_algorithmic_bytes": int(avg_bytes)},
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(s, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
