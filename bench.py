"""Decode GEMV benchmark.  Prints one JSON line (rank 0, N=1).

Default workload (``--workload stream``): one step = one token's pass over
the Qwen2-7B-shaped 28-layer W4A8 weight stream plus the int4 lm_head, all
resident in HBM: 113 linears (28 layers x {fused QKV, O, fused gate/up, down}
+ lm_head), by default one launch of the persistent pass (``--per-linear``:
one fused launch per linear).  Each linear quantises its activation per token
in the prologue, takes INT4 x INT8 dot products into exact int32 and applies
the fp32 epilogue.

Other workloads (each one JSON line of the same form):
  single  one Q-projection linear [3584, 3584], 1 % outliers in x
  layer   one decoder layer (fused QKV, O, fused gate/up, down)
  gemma   35 Gemma-shaped group-32 layers (fp16 x) + the W8A16 lm_head
  verify  the M-token verify GEMM over [18944, 3584] and [3584, 18944],
          M in --verify-m (default 1,2,4,8,16)
Weights that fit the Infinity Cache rotate through a >= 1 GB pool of copies.
Per-linear launches are captured once into a HIP graph and replayed
(``--eager``: launched from Python every step).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload ...]
"""
import argparse
import hashlib
import json
import os
import re
import struct
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for W4A8 decode GEMV; implied 28-layer tok/s"
HBM_PEAK_GBS = 8000.0
WORKLOADS = ("stream", "single", "layer", "gemma", "verify", "chain", "int8x", "shard")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", choices=WORKLOADS, default="stream")
    p.add_argument("--layers", type=int, default=0, help="decoder layers (0 = the model's: 28 / 35)")
    p.add_argument("--r", type=int, default=0, help="rows per lane group (0 = automatic)")
    p.add_argument("--lanes", type=int, default=0, help="lanes per row (0 = automatic)")
    p.add_argument("--per-linear", action="store_true",
                   help="stream / layer: one launch per linear instead of the persistent pass")
    p.add_argument("--eager", action="store_true",
                   help="launch per-linear kernels from Python each step instead of replaying "
                        "them from a captured HIP graph")
    p.add_argument("--w4a16", action="store_true",
                   help="stream: the float-unpack comparison (gemv_w4a16 per linear, fp16 x) "
                        "instead of the W4A8 path")
    p.add_argument("--lm-head", choices=("w8a16", "q6k"), default="w8a16",
                   help="gemma: the lm_head form in the token step (int8-expanded or packed 6-bit)")
    p.add_argument("--verify-m", default="1,2,4,8,16")
    p.add_argument("--impl", type=int, default=0,
                   help="verify kernel: 0 automatic, 1 dot4, 2 MFMA per tile, 3 MFMA balanced blocks")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="before the timed region, run one plain device copy of this many MiB "
                        "(the reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--weights-cache", default="", metavar="PATH",
                   help="stream workload: copy the weights and activations from PATH (safetensors) when it "
                        "holds this stream, else generate them and write PATH; a run that loads it launches "
                        "none of the generator's kernels")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    return p.parse_args()


# Counter summaries (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated) of
# each workload's dominant kernel, at the configuration the file names.
TRAFFIC = {w: os.path.join(ROOT, "profiles", f) for w, f in (
    ("stream", "k_decode_pass_qwen2-7b-28L_traffic.md"),
    ("layer", "k_decode_pass_qwen2-7b-layer-pool_traffic.md"),
    ("single", "k_linear_wide_single-q-proj-3584x3584_traffic.md"),
    ("verify", "k_verify_blocks_verify-18944x3584-M16_traffic.md"),
    ("gemma", "k_gemv_w8a16_g32_gemma-lm-head_traffic.md"))}
TRAFFIC_SUMMARY = TRAFFIC["stream"]


def _elf_sections(b):
    """Section headers of a little-endian ELF64 image: name, type, address,
    file offset, size, link."""
    shoff = struct.unpack_from("<Q", b, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, 0x3A)
    secs = []
    for i in range(shnum):
        name, typ, _, addr, off, size, link = struct.unpack_from("<IIQQQQI", b, shoff + i * shentsize)
        secs.append({"name": name, "type": typ, "addr": addr, "off": off, "size": size, "link": link})
    names = secs[shstrndx]["off"]
    for sec in secs:
        sec["name"] = b[names + sec["name"]:b.index(b"\0", names + sec["name"])].decode()
    return secs


def kernel_code_sha256(lib_path, needle="k_decode_pass", arch="gfx950", exact=False):
    """sha256 of a kernel's machine code in the library's ``arch`` code
    object (the clang offload bundle in .hip_fatbin, then the symbol whose
    name contains ``needle``, or is ``needle`` when ``exact``), or None if it
    cannot be found."""
    try:
        b = open(lib_path, "rb").read()
        fb = [sec for sec in _elf_sections(b) if sec["name"] == ".hip_fatbin"][0]
        d = b[fb["off"]:fb["off"] + fb["size"]]
        if d[:24] != b"__CLANG_OFFLOAD_BUNDLE__":
            return None
        n, p, co = struct.unpack_from("<Q", d, 24)[0], 32, None
        for _ in range(n):
            off, size, tl = struct.unpack_from("<QQQ", d, p)
            triple = d[p + 24:p + 24 + tl].decode()
            p += 24 + tl
            if arch in triple:
                co = d[off:off + size]
        secs = _elf_sections(co)
        for sym in (sec for sec in secs if sec["type"] in (2, 11)):   # SHT_SYMTAB, SHT_DYNSYM
            strs = secs[sym["link"]]["off"]
            for i in range(sym["size"] // 24):
                nm, info, _, _, val, size = struct.unpack_from("<IBBHQQ", co, sym["off"] + 24 * i)
                name = co[strs + nm:co.index(b"\0", strs + nm)].decode()
                if (name == needle if exact else needle in name) and (info & 0xF) == 2 and size:  # STT_FUNC
                    text = [sec for sec in secs if sec["type"] == 1 and sec["addr"] <= val < sec["addr"] + sec["size"]][0]
                    start = text["off"] + val - text["addr"]
                    return hashlib.sha256(co[start:start + size]).hexdigest()
    except (OSError, IndexError, struct.error, TypeError, ValueError):
        return None
    return None


def measured_traffic(summary=TRAFFIC_SUMMARY):
    """HBM bytes per launch from a committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary (copy-calibrated), or None unless the library in use holds the
    same machine code for the summary's kernel (``kernel_symbol``, else
    k_decode_pass) as the one the counters were taken on."""
    from bit_quantized_decode_quantize_amd import bqd
    try:
        text = open(summary, encoding="utf-8").read()
    except OSError:
        return None
    vals = dict(re.findall(r"^(traffic_bytes_per_launch|kernel_code_sha256|kernel_symbol): (\S+)$", text, re.M))
    if "kernel_symbol" in vals:
        sha = kernel_code_sha256(bqd.LIB_PATH, vals["kernel_symbol"], exact=True)
    else:
        sha = kernel_code_sha256(bqd.LIB_PATH)
    if sha is None or vals.get("kernel_code_sha256") != sha or "traffic_bytes_per_launch" not in vals:
        return None
    return int(vals["traffic_bytes_per_launch"])


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# --------------------------------------------------------------- timing ---
def time_steps(step, steps, warmup, graph_steps=0):
    """Mean ms per step over ``steps`` steps on the current stream, events
    around the whole region.  graph_steps > 0: capture that many consecutive
    steps into one HIP graph and replay it ceil(steps / graph_steps) times.
    Returns (ms_per_step, steps actually timed)."""
    import torch
    st = torch.cuda.current_stream()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if graph_steps:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(graph_steps):
                step()
        torch.cuda.synchronize()
        g.replay()  # warm replay
        torch.cuda.synchronize()
        reps = max(1, -(-steps // graph_steps))
        run, n = (lambda: g.replay()), reps * graph_steps
        calls = reps
    else:
        run, n, calls = step, steps, steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(calls):
        run()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n, n


def repeat_spread(step, steps, reps=5):
    """ms per step over ``reps`` further regions of ``steps`` steps each:
    median, min and max (the timed region above is the reported value)."""
    import statistics
    import torch
    st = torch.cuda.current_stream()
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(steps):
            step()
        e1.record(st)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return {"reps": reps, "steps_each": steps, "median": round(statistics.median(out), 5),
            "min": round(min(out), 5), "max": round(max(out), 5)}


def read_ceiling(dev, nbytes=2 << 30):
    """Best bandwidth of the library's streaming-read kernel over a few launch
    shapes, reading a 2 GiB buffer (8x the Infinity Cache) per launch."""
    import torch
    from bit_quantized_decode_quantize_amd import bqd
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1 << 14, dtype=torch.int32, device=dev)
    best, shape = 0.0, None
    for unroll, grid in ((1, 1024), (1, 2048), (1, 4096), (4, 512), (4, 1024), (8, 256), (8, 512)):
        bqd.read_probe(buf, sink, grid, unroll)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            bqd.read_probe(buf, sink, grid, unroll)
        e1.record()
        torch.cuda.synchronize()
        gbs = 5 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
        if gbs > best:
            best, shape = gbs, (unroll, grid)
    del buf
    torch.cuda.empty_cache()
    return {"GB/s": round(best, 1), "kernel": "read_probe", "unroll": shape[0], "grid": shape[1],
            "bytes_per_launch": nbytes}


def roofline(achieved_gbs, kernel, avg_us, avg_bytes, traffic=None):
    return {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
            "avg_launch_us": round(avg_us, 3), "avg_algorithmic_bytes": int(avg_bytes)}


def inputs_digest(*tensors, nbytes=1 << 20):
    """First 16 hex digits of a sha256 over the first ``nbytes`` bytes of each
    tensor (copied to the host), in order: names the seeded synthetic inputs
    a line ran on, so two runs can be seen to have used the same data."""
    import torch
    h = hashlib.sha256()
    for t in tensors:
        if t is None:
            continue
        b = t.detach().contiguous().reshape(-1).view(torch.uint8)[:nbytes]
        h.update(b.cpu().numpy().tobytes())
    return h.hexdigest()[:16]


def base_line(a, value, ms, steps, config, dtype="int8"):
    return {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": dtype, "data": "synthetic", "config": config,
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2)}


def cold_call_us(step, dev, reps=5):
    """One call after 512 MiB of writes have flushed the caches, events
    around the call alone; median of ``reps``.  The events and the call are
    enqueued while the flush still runs, so host-side launch cost is not
    counted."""
    import statistics
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    t = []
    for i in range(reps):
        torch.cuda.synchronize()
        flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) * 1e3)
    del flush
    return round(statistics.median(t), 2)


def host_facts():
    """The host the CPU baseline ran on: logical CPUs, the CPUs this process
    may use, and the CPU model."""
    model = ""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpus_allowed": len(os.sched_getaffinity(0)), "cpu_model": model}


HOST = {}


def cpu_loop(fn, sample_bytes, seconds):
    """Runs fn repeatedly for about ``seconds`` on one core: the calling
    thread (which runs the single-threaded C oracle) is pinned to the first
    CPU it may use, and its previous affinity restored afterwards."""
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    HOST.update(host_facts(), pinned_core=core)
    os.sched_setaffinity(0, {core})
    try:
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return sample_bytes * reps / el / 1e9, reps, el
    finally:
        os.sched_setaffinity(0, allowed)


# ------------------------------------------------------------ workloads ---
def run_stream(a, dev):
    import torch
    from bit_quantized_decode_quantize_amd import bqd
    from bit_quantized_decode_quantize_amd import decode_stream as DS

    layers = a.layers or 28
    t0 = time.time()
    s = DS.QwenW4A8Stream(layers=layers, device=dev, r=a.r, lanes_per_row=a.lanes,
                          persistent=not (a.per_linear or a.w4a16), cache=a.weights_cache or None)
    if a.w4a16:
        return run_stream_w4a16(a, dev, s, layers)
    log(f"stream built: {len(s.linears)} linears, {s.weight_bytes() / 1e9:.3f} GB packed, "
        f"{time.time() - t0:.1f} s ({'copied from ' + a.weights_cache if s.cached else 'generated'})")
    if a.weights_cache and not s.cached:
        t0 = time.time()
        s.save(a.weights_cache)
        log(f"stream written to {a.weights_cache}, {time.time() - t0:.1f} s")
    st = torch.cuda.current_stream()

    graph_steps = 1 if ((not a.eager) and a.per_linear) else 0
    step_bytes = s.bytes_per_step()
    if s.persistent:
        # The decoder's data flow: each linear reads the previous linear's
        # output (a prefix where the previous linear is wider), so every
        # linear waits for the one before it.  One launch per step carries
        # every byte; a second pass of the same K steps with events around
        # each launch gives the kernel's own duration.
        cp = s.chained_pass()
        step = cp.run
        ms, n = time_steps(step, a.steps, a.warmup, 0)
        evs = []
        for _ in range(a.steps):
            b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            b0.record(st)
            step()
            b1.record(st)
            evs.append((b0, b1))
        torch.cuda.synchronize()
        if cp.error_word():
            raise RuntimeError(f"chained pass reported a wait time-out (error word {cp.error_word()})")
        dur_us = [b0.elapsed_time(b1) * 1e3 for b0, b1 in evs]
        avg_us, avg_bytes = sum(dur_us) / len(dur_us), step_bytes
        kernel = f"k_decode_pass (persistent: whole token pass, {len(s.linears)} chained linears, one launch)"
        traffic = measured_traffic() if layers == 28 else None
        # The same linears with independent activations written before the
        # launch: nothing to wait for, the pass streams (an upper bound).
        ims, _ = time_steps(s.step, a.steps, a.warmup, 0)
        if s.pass_.error_word():
            raise RuntimeError(f"independent pass reported an error (error word {s.pass_.error_word()})")
        independent = {"ms_per_step": round(ims, 5), "GB/s": round(step_bytes / (ims * 1e-3) / 1e9, 1),
                       "tok_per_s": round(1e3 / ims, 2),
                       "note": "the same linears, each with its own activation written before the launch: "
                               "no dependency between linears"}
        # The dependency alone: as many chained linears, [64, 64] each.
        fp = s.link_floor_pass(64)
        fms, _ = time_steps(fp.run, a.steps, a.warmup, 0)
        if fp.error_word():
            raise RuntimeError(f"link-floor pass reported a wait time-out (error word {fp.error_word()})")
        link_floor = {"ms_per_step": round(fms, 5), "us_per_linear": round(fms * 1e3 / len(s.linears), 3),
                      "note": f"{len(s.linears)} chained [64, 64] linears: output store, poll, activation "
                              "staging and a few rows per dependency, next to no weight traffic"}
        del fp
    else:
        step = s.step
        ms, n = time_steps(step, a.steps, a.warmup, graph_steps)
        # Dominant kernel: the gate/up linears + lm_head (most of the bytes),
        # each launch bracketed by events in a second eager pass.
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
        avg_us, avg_bytes = sum(dur_us) / len(dur_us), sum(dom_bytes) / len(dom_bytes)
        kernel = "k_gemv_w4a8 (fused gate/up linears and lm_head, one launch per linear)"
        traffic = None
    gbs = step_bytes / (ms * 1e-3) / 1e9
    achieved = avg_bytes / (avg_us * 1e-6) / 1e9
    launch = "persistent pass" if s.persistent else ("per-linear, HIP graph" if graph_steps else "per-linear")
    flow = ("chained: linear i reads linear i-1's output" if s.persistent
            else "each linear's activation written before the step")
    out = base_line(a, gbs, ms, n, {
        "workload": f"qwen2-7b-shaped {layers}-layer W4A8 decode weight stream + int4 lm_head "
                    "(per-row scales, fused QKV and gate/up, fused act-quant)",
        "activations": flow,
        "launch": launch, "layers": layers, "hidden": 3584, "kv_dim": 512, "intermediate": 18944,
        "vocab": 152064, "global_batch": 1, "parallelism": "none",
        "bytes_per_step": step_bytes, "packed_weight_bytes": s.weight_bytes()})
    out["tok_per_s"] = round(1e3 / ms, 2)
    out["us_per_gemv"] = round(ms * 1e3 / len(s.linears), 3)
    d0, dl = s.linears[0], s.linears[-1]
    out["inputs_sha256"] = inputs_digest(d0["wq"], d0["sw"], d0["b"], d0["x"], dl["wq"], dl["sw"], dl["x"])
    out["ms_per_step_spread"] = repeat_spread(step, max(1, a.steps // 5))
    out["roofline"] = roofline(achieved, kernel, avg_us, avg_bytes, traffic)
    if s.persistent:
        out["independent"] = independent
        out["link_floor"] = link_floor
    ceil = read_ceiling(dev)
    out["read_ceiling"] = ceil
    out["pct_of_read_ceiling"] = round(100.0 * gbs / ceil["GB/s"], 2)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_stream(s, a.cpu_seconds)
    return out


def run_stream_w4a16(a, dev, s, layers):
    """The same 28-layer weights through the float-unpack comparison GEMV
    (fp16 x, one graph-replayed launch per linear)."""
    import torch
    from bit_quantized_decode_quantize_amd import bqd
    x16 = [d["x"].to(torch.float16) for d in s.linears]

    def step():
        for d, x in zip(s.linears, x16):
            bqd.gemv_w4a16(d["wq"], d["sw"], d["b"], x, y=d["y"], r=a.r, lanes_per_row=a.lanes)
    ms, n = time_steps(step, a.steps, a.warmup, 0 if a.eager else 1)
    step_bytes = sum(d["N"] * d["K"] // 2 + 4 * d["N"] + (4 * d["N"] if d["b"] is not None else 0) + 2 * d["K"]
                     + 4 * d["N"] for d in s.linears)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    out = base_line(a, gbs, ms, n, {
        "workload": f"qwen2-7b-shaped {layers}-layer stream through the W4A16 float-unpack comparison GEMV "
                    "(fp16 x, per-row int4)", "launch": "per-linear, HIP graph" if not a.eager else "per-linear",
        "layers": layers, "bytes_per_step": step_bytes}, dtype="fp16")
    out["tok_per_s"] = round(1e3 / ms, 2)
    out["roofline"] = roofline(gbs, "k_gemv_w4a16 (every linear, one launch each)", ms * 1e3 / len(s.linears),
                               step_bytes / len(s.linears))
    return out


def cpu_baseline_stream(stream, seconds):
    """The C oracle, single-threaded on this host, over layer 0 of the same
    stream (its four linears: activation quantisation + GEMV), repeated for
    about ``seconds``; reported as algorithmic GB/s and implied tok/s."""
    import torch
    import oracle as O
    from bit_quantized_decode_quantize_amd import decode_stream as DS

    work = []
    for d in stream.linears[:4]:
        W = stream.fp32_rows(d, torch.arange(d["N"])).cpu().numpy()
        w, s = O.prepare_int4_rowwise(W)
        del W
        b = None if d["b"] is None else d["b"].cpu().numpy()
        work.append((w, s, b, d["x"].cpu().numpy(), DS.algorithmic_bytes_linear(d["N"], d["K"], b is not None)))
    sample_bytes = sum(wk[4] for wk in work)

    def once():
        for w, s, b, x, _ in work:
            O.linear_w4a8(w, s, b, x)
    gbs, reps, el = cpu_loop(once, sample_bytes, seconds)
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle", "host": dict(HOST),
            "sample": f"layer 0 of the stream (fused QKV, O, gate/up, down: {sample_bytes} algorithmic bytes), "
                      f"{reps} passes in {el:.1f} s, single-threaded C; implied tok/s over the full "
                      f"stream {gbs * 1e9 / stream.bytes_per_step():.4f}"}


def run_single(a, dev):
    import torch
    from bit_quantized_decode_quantize_amd import workloads as WL
    from bit_quantized_decode_quantize_amd import inputs as I

    w = WL.SingleGemvPool(device=dev, r=a.r, lanes_per_row=a.lanes)
    log(f"single GEMV pool: {w.copies} copies of {w.weight_bytes()} B")
    ms, n = time_steps(w.step, a.steps, a.warmup, w.copies if (not a.eager) else 0)
    gbs = w.bytes_per_step() / (ms * 1e-3) / 1e9
    out = base_line(a, gbs, ms, n, {
        "workload": "single W4A8 linear (Q projection) [3584, 3584], per-row int4, x fp32 with 1% x20 "
                    "outliers, fused act-quant", "launch": "HIP graph" if (not a.eager) else "eager",
        "N": w.N, "K": w.K, "rotation_copies": w.copies, "bytes_per_step": w.bytes_per_step()})
    out["us_per_gemv"] = round(ms * 1e3, 3)
    out["inputs_sha256"] = inputs_digest(w.wq[0], w.sw[0], w.b[0], w.x)
    out["cold_single_call_us"] = cold_call_us(w.step, dev)
    # The float-unpack comparison (W4A16) on the same weights, fp16 x.
    from bit_quantized_decode_quantize_amd import bqd
    x16 = w.x.to(torch.float16)
    state = {"i": 0}

    def step16():
        c = state["i"] % w.copies
        state["i"] += 1
        bqd.gemv_w4a16(w.wq[c], w.sw[c], w.b[c], x16, y=w.y, r=a.r, lanes_per_row=a.lanes)
    ms16, _ = time_steps(step16, a.steps, a.warmup, w.copies if (not a.eager) else 0)
    out["w4a16_us_per_gemv"] = round(ms16 * 1e3, 3)
    # The same GEMV on int8 codes a producer already wrote (RMSNorm or SwiGLU
    # fused with the quantisation): the activation is quantised once here,
    # outside the timed region, and each call reads the codes and s^x.
    qx, sx = bqd.quantize_act(w.x)

    def step_q8():
        c = state["i"] % w.copies
        state["i"] += 1
        bqd.gemv_w4a8(w.wq[c], w.sw[c], w.b[c], qx, sx, y=w.y, r=a.r, lanes_per_row=a.lanes)
    ms_q8, _ = time_steps(step_q8, a.steps, a.warmup, w.copies if (not a.eager) else 0)
    out["int8_x_us_per_gemv"] = round(ms_q8 * 1e3, 3)
    out["int8_x_note"] = ("x quantised by its producer (not timed here): the GEMV alone on int8 codes and s^x, "
                          "k_linear_wide<2, X_Q8>")
    auto = not (a.r or a.lanes)
    kname = ("k_linear_wide<2, X_F32, 512> (fused linear, one 512-thread workgroup per 8 rows, one launch per step)"
             if auto else "k_gemv_w4a8 (fused linear, one launch per step)")
    out["roofline"] = roofline(gbs, kname, ms * 1e3, w.bytes_per_step(),
                               measured_traffic(TRAFFIC["single"]) if auto else None)
    if not a.no_cpu_baseline:
        import oracle as O
        d = I.single_gemv_inputs(0, "cpu")
        wq, sw = O.prepare_int4_rowwise(d["W"].numpy())
        x, b = d["x"].numpy(), d["b"].numpy()
        g, reps, el = cpu_loop(lambda: O.linear_w4a8(wq, sw, b, x), w.bytes_per_step(), a.cpu_seconds)
        out["cpu_baseline"] = {"value": round(g, 3), "unit": "GB/s", "cores": 1, "kind": "oracle", "host": dict(HOST),
                               "sample": f"the same linear, {reps} calls in {el:.1f} s, single-threaded C"}
    return out


def run_layer(a, dev):
    from bit_quantized_decode_quantize_amd import workloads as WL

    w = WL.LayerPool(device=dev, persistent=not a.per_linear)
    log(f"layer pool: {w.copies} copies of {w.weight_bytes()} B")
    if w.persistent:
        ms_call, n = time_steps(w.step, max(1, a.steps // w.copies), a.warmup)
        ms, n = ms_call / w.steps_per_call, n * w.steps_per_call
        kernel = f"k_decode_pass (persistent: {w.copies} layers = {4 * w.copies} linears per launch)"
        avg_us, avg_bytes = ms_call * 1e3, w.bytes_per_step() * w.steps_per_call
    else:
        ms, n = time_steps(w.step, a.steps, a.warmup, w.copies if (not a.eager) else 0)
        kernel = "k_gemv_w4a8 (4 fused linears per layer, one launch each)"
        avg_us, avg_bytes = ms * 1e3 / 4, w.bytes_per_step() / 4
    gbs = w.bytes_per_step() / (ms * 1e-3) / 1e9
    launch = "persistent pass" if w.persistent else ("per-linear, HIP graph" if (not a.eager) else "per-linear")
    out = base_line(a, gbs, ms, n, {
        "workload": "one qwen2-7b-shaped decoder layer: fused QKV [4608,3584], O [3584,3584], fused gate/up "
                    "[37888,3584], down [3584,18944], per-row int4, fused act-quant",
        "launch": launch, "rotation_copies": w.copies, "bytes_per_step": w.bytes_per_step()})
    out["us_per_layer"] = round(ms * 1e3, 3)
    out["implied_28_layer_gemv_us"] = round(28 * ms * 1e3, 1)
    out["inputs_sha256"] = inputs_digest(*[t for e in w.layers[0] for t in (e["wq"], e["sw"], e["b"], e["x"])])
    out["roofline"] = roofline(avg_bytes / (avg_us * 1e-6) / 1e9, kernel, avg_us, avg_bytes,
                               measured_traffic(TRAFFIC["layer"]) if w.persistent else None)
    if not a.no_cpu_baseline:
        import oracle as O
        from bit_quantized_decode_quantize_amd import decode_stream as DS
        work = []
        for e in w.layers[0]:
            W = DS.linear_weight_fp32("qwen/L0", e["name"], 0, dev).cpu().numpy()
            wq, sw = O.prepare_int4_rowwise(W)
            del W
            work.append((wq, sw, e["b"].cpu().numpy(), e["x"].cpu().numpy()))
        g, reps, el = cpu_loop(lambda: [O.linear_w4a8(*t) for t in work], w.bytes_per_step(), a.cpu_seconds)
        out["cpu_baseline"] = {"value": round(g, 3), "unit": "GB/s", "cores": 1, "kind": "oracle", "host": dict(HOST),
                               "sample": f"the same layer, {reps} passes in {el:.1f} s, single-threaded C"}
    return out


def run_shard(a, dev):
    """One GPU's share of the Qwen2-7B-shaped layer under 8-way tensor
    parallelism, at its real shapes: QKV and gate/up by output rows, O and
    down by K slices with int32 partial accumulators (the collectives that
    would join the shares are not part of a one-GPU run)."""
    from bit_quantized_decode_quantize_amd import workloads as WL

    w = WL.ShardLayerPool(device=dev, G=8, rank=0)
    log(f"shard pool: {w.copies} copies of {w.weight_bytes()} B")
    graph = w.copies if (not a.eager) else 0
    ms, n = time_steps(w.step, a.steps, a.warmup, graph)
    gbs = w.bytes_per_step() / (ms * 1e-3) / 1e9
    shapes = ", ".join(f"{e['name']} {'rows' if e['kind'] == 'rows' else 'K slice'} [{e['N']}, {e['K']}]"
                       for e in w.layers[0])
    out = base_line(a, gbs, ms, n, {
        "workload": f"one GPU's share (rank 0 of 8) of a qwen2-7b-shaped decoder layer under tensor parallelism: "
                    f"{shapes}; per-row int4, fused act-quant on the row shares, int32 partials on the K slices",
        "launch": "per-linear, HIP graph" if graph else "per-linear", "tp_degree": w.G, "rank": w.rank,
        "rotation_copies": w.copies, "bytes_per_step": w.bytes_per_step()})
    out["us_per_share_layer"] = round(ms * 1e3, 3)
    per = []
    for j, e0 in enumerate(w.layers[0]):
        state = {"i": 0}

        def one(j=j):
            WL.ShardLayerPool.run_linear(w.layers[state["i"] % w.copies][j])
            state["i"] += 1
        ms_j, _ = time_steps(one, a.steps, a.warmup, graph)
        nb = WL.ShardLayerPool.linear_bytes(e0)
        per.append({"name": e0["name"], "split": "rows" if e0["kind"] == "rows" else "K", "N": e0["N"],
                    "K": e0["K"], "us": round(ms_j * 1e3, 3), "GB/s": round(nb / (ms_j * 1e-3) / 1e9, 1),
                    "bytes": nb})
    out["linears"] = per
    out["inputs_sha256"] = inputs_digest(*[t for e in w.layers[0] for t in (e["wq"], e["sw"])])
    g = next(d for d in per if d["name"] == "gate_up")
    out["roofline"] = roofline(g["GB/s"], "k_linear_wide<2, X_F32> (the gate/up row share, fused act-quant, "
                               "one launch)", g["us"], g["bytes"], None)
    if not a.no_cpu_baseline:
        import oracle as O
        from bit_quantized_decode_quantize_amd import decode_stream as DS
        work = []
        acts = DS.layer_inputs("qwen/L0", 0, dev)
        for e in w.layers[0]:
            W = DS.linear_weight_fp32("qwen/L0", e["name"], 0, dev)
            if e["kind"] == "rows":
                rows = WL.shard_row_index(e["name"], w.rank, w.G, dev)
                wq, sw = O.prepare_int4_rowwise(W[rows].cpu().numpy())
                work.append(("rows", wq, sw, e["b"].cpu().numpy(), e["x"].cpu().numpy()))
            else:
                wq, sw = O.prepare_int4_rowwise(W.cpu().numpy())
                qx, sx = O.quantize_act(acts[e["name"]].cpu().numpy())
                k0, ks = e["k0"], e["K"]
                work.append(("k", wq[:, k0 // 8:(k0 + ks) // 8].copy(), sw, float(sx), qx[k0:k0 + ks].copy()))
            del W

        def once():
            for kind, wq, sw, b_or_sx, x in work:
                if kind == "rows":
                    O.linear_w4a8(wq, sw, b_or_sx, x)
                else:
                    O.gemv_w4a8(wq, sw, None, x, b_or_sx)
        g_cpu, reps, el = cpu_loop(once, w.bytes_per_step(), a.cpu_seconds)
        out["cpu_baseline"] = {"value": round(g_cpu, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "host": dict(HOST),
                               "sample": f"the same share, {reps} passes in {el:.1f} s, single-threaded C"}
    return out


def run_gemma(a, dev):
    from bit_quantized_decode_quantize_amd import workloads as WL
    from bit_quantized_decode_quantize_amd import inputs as I

    layers = a.layers or 35
    t0 = time.time()
    w = WL.GemmaG32Stream(layers=layers, device=dev, r=a.r, lanes_per_row=a.lanes, head=a.lm_head)
    log(f"gemma stream built: {w.launches_per_step} launches, {w.weight_bytes() / 1e9:.3f} GB, "
        f"{time.time() - t0:.1f} s")
    # The token step: the 140 group-32 linears chained in one persistent
    # pass (each reads the previous output), then the lm_head (--per-linear:
    # one graph-replayed launch per linear, each with its own activation).
    if a.per_linear:
        step, step_bytes = w.step, w.bytes_per_step()
        ms, n = time_steps(step, a.steps, a.warmup, 1 if (not a.eager) else 0)
    else:
        gp = w.make_pass(chained=True)

        def step():
            gp.run()
            w.run_head()
        step_bytes = w.pass_bytes(chained=True)
        ms, n = time_steps(step, a.steps, a.warmup, 0)
        if gp.error_word():
            raise RuntimeError(f"gemma pass reported an error (error word {gp.error_word()})")
        ip = w.make_pass(chained=False)

        def istep():
            ip.run()
            w.run_head()
        ims, _ = time_steps(istep, a.steps, a.warmup, 0)
        pms, _ = time_steps(w.step, a.steps, a.warmup, 1)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    # Both lm_head forms alone (the largest single matrix), back to back.
    heads = {}
    for kind, fn in (("w8a16", w.lm_head), ("q6k", w.lm_head_q6k)):
        ms_h, _ = time_steps(fn, max(20, a.steps), 2, 0)
        heads[kind] = {"us": round(ms_h * 1e3, 2), "bytes": w.head_bytes(kind),
                       "GB/s": round(w.head_bytes(kind) / (ms_h * 1e-3) / 1e9, 1)}
    head_form = {"w8a16": "W8A16 lm_head [262144,1536] (int8 in [-32,31], fp16 group-32 scales)",
                 "q6k": "packed 6-bit lm_head [262144,1536] (210 B per 256 weights, decoded in registers)"}
    launch = ("per-linear, HIP graph" if (not a.eager) else "per-linear") if a.per_linear else \
        "persistent pass (140 chained linears) + lm_head launch"
    out = base_line(a, gbs, ms, n, {
        "workload": f"gemma-shaped {layers}-layer Q4_0-style group-32 W4A8 stream + " + head_form[a.lm_head],
        "activations": ("each linear's own fp16 activation" if a.per_linear else
                        "chained: linear i reads linear i-1's fp32 output"),
        "launch": launch, "layers": layers,
        "bytes_per_step": step_bytes, "weight_bytes": w.weight_bytes()}, dtype="int8+fp16")
    out["tok_per_s"] = round(1e3 / ms, 2)
    out["us_per_gemv"] = round(ms * 1e3 / w.launches_per_step, 3)
    out["inputs_sha256"] = inputs_digest(w.linears[0]["wq"], w.linears[0]["s16"], w.linears[0]["x"],
                                         w.linears[-1]["wq"], w.linears[-1]["s16"])
    if not a.per_linear:
        ib = w.pass_bytes(chained=False)
        out["independent"] = {"ms_per_step": round(ims, 5), "GB/s": round(ib / (ims * 1e-3) / 1e9, 1),
                              "note": "the same pass with each linear's own fp16 activation (no dependency)"}
        out["per_linear_graph"] = {"ms_per_step": round(pms, 5),
                                   "GB/s": round(w.bytes_per_step() / (pms * 1e-3) / 1e9, 1),
                                   "note": "one graph-replayed launch per linear, own fp16 activations"}
    out["lm_head"] = heads[a.lm_head]
    out["lm_head_forms"] = heads
    h = heads[a.lm_head]
    kern = {"w8a16": "k_gemv_w8a16_g32", "q6k": "k_gemv_q6k"}[a.lm_head]
    out["roofline"] = roofline(h["GB/s"], f"{kern} (lm_head, largest single launch)", h["us"], h["bytes"],
                               measured_traffic(TRAFFIC["gemma"]) if a.lm_head == "w8a16" else None)
    if not a.no_cpu_baseline:
        import oracle as O
        work = []
        for d in w.linears[:4]:
            W = I.normal(f"gemma/L0/{d['name']}/W", (d["N"], d["K"]), 0.02, 0, dev).cpu().numpy()
            wq, s16 = O.prepare_int4_group32(W)
            del W
            work.append((wq, s16, None, d["x"].cpu().numpy()))
        sample = sum(WL.bytes_group32_linear(d["N"], d["K"], False) for d in w.linears[:4])
        g, reps, el = cpu_loop(lambda: [O.linear_w4a8_group32(*t) for t in work], sample, a.cpu_seconds)
        out["cpu_baseline"] = {"value": round(g, 3), "unit": "GB/s", "cores": 1, "kind": "oracle", "host": dict(HOST),
                               "sample": f"layer 0 of the stream (4 group-32 linears, {sample} B), {reps} "
                                         f"passes in {el:.1f} s, single-threaded C"}
    return out


def run_verify(a, dev):
    import torch
    from bit_quantized_decode_quantize_amd import workloads as WL

    ms_list = [int(m) for m in a.verify_m.split(",")]
    sweep = []
    for N, K in ((18944, 3584), (3584, 18944)):
        for M in ms_list:
            w = WL.VerifyPool(N, K, M, device=dev, impl=a.impl)
            ms, n = time_steps(w.step, max(a.steps, 2 * w.copies), a.warmup, w.copies if (not a.eager) else 0)
            sweep.append({"N": N, "K": K, "M": M, "us": round(ms * 1e3, 3),
                          "GB/s": round(w.bytes_per_step() / (ms * 1e-3) / 1e9, 1),
                          "Tops": round(w.int_ops_per_step() / (ms * 1e-3) / 1e12, 2),
                          "rotation_copies": w.copies, "steps": n})
            log(f"verify {N}x{K} M={M}: {sweep[-1]}")
            if N == 18944:
                digest = inputs_digest(w.wq[0], w.sw[0], w.b[0], w.qx, w.sx)
            del w
            torch.cuda.empty_cache()
    # A1 on its own: the per-token activation quantisation that feeds the
    # verify GEMM (M tokens, fp32 X), graph-replayed, x read once per call.
    from bit_quantized_decode_quantize_amd import bqd, inputs as I
    qa = []
    for K in (3584, 18944):
        for M in ms_list:
            X = I.normal(f"verify/quant/{M}x{K}", (M, K), 1.0, 0, dev)
            qx = torch.empty(M, K, dtype=torch.int8, device=dev)
            sx = torch.empty(M, dtype=torch.float32, device=dev)
            ms, n = time_steps(lambda: bqd.quantize_act(X, qx=qx, sx=sx), max(a.steps, 64), a.warmup,
                               0 if a.eager else 16)
            qa.append({"K": K, "M": M, "us": round(ms * 1e3, 3)})
            del X, qx, sx
    log(f"quantize_act: {qa}")
    last = max((r for r in sweep if r["N"] == 18944), key=lambda r: r["M"])
    ms = last["us"] * 1e-3
    out = base_line(a, last["GB/s"], ms, last["steps"], {
        "workload": "M-token verify GEMM, per-row int4 weights [18944,3584] and [3584,18944], int8 X [M,K] "
                    "(per-token scales), bias", "impl": a.impl, "M": ms_list})
    out["sweep"] = sweep
    out["inputs_sha256"] = digest  # the [18944, 3584] pool at the largest M
    out["quantize_act"] = qa
    out["quantize_act_note"] = ("graph-replayed calls on one resident X (L2-resident after the first): "
                                "per-call latency, not a bandwidth")
    wl_bytes = WL.bytes_verify(last["M"], 18944, 3584)
    kname = ("k_gemv_w4a8" if last["M"] == 1 and a.impl == 0 else
             "k_verify_w4a8" if a.impl == 1 else "k_verify_mfma" if a.impl == 2 else "k_verify_blocks")
    out["roofline"] = roofline(last["GB/s"], f"{kname} (M={last['M']}, [18944,3584], one launch per step)",
                               last["us"], wl_bytes,
                               measured_traffic(TRAFFIC["verify"]) if (last["M"] == 16 and a.impl == 0) else None)
    if not a.no_cpu_baseline:
        import oracle as O
        from bit_quantized_decode_quantize_amd import inputs as I
        N, K, M = 18944, 3584, last["M"]
        W = I.normal(f"verify/{N}x{K}/W", (N, K), 0.02, 0, dev).cpu().numpy()
        wq, sw = O.prepare_int4_rowwise(W)
        del W
        b = I.normal(f"verify/{N}x{K}/b", N, 0.01, 0, dev).cpu().numpy()
        X = I.normal(f"verify/{N}x{K}/X", (M, K), 1.0, 0, dev).cpu().numpy()
        qx, sx = O.quantize_act(X)
        g, reps, el = cpu_loop(lambda: O.gemm_w4a8_verify(wq, sw, b, qx, sx), wl_bytes, a.cpu_seconds)
        out["cpu_baseline"] = {"value": round(g, 3), "unit": "GB/s", "cores": 1, "kind": "oracle", "host": dict(HOST),
                               "sample": f"verify [18944,3584] at M={M}, {reps} calls in {el:.1f} s, "
                                         "single-threaded C"}
    return out


def run_chain(a, dev):
    """The 28-layer stream wired into a decoder's data flow with the
    activation producers (residual add + RMSNorm, SwiGLU) fused with the
    quantisation, one HIP graph per token.  Timed three ways that give the
    same logits: producers writing int8 codes (the value), RMSNorm +
    quantisation in the consuming linear's prologue, and fp32 producers with
    linears that quantise in their prologue."""
    import torch
    from bit_quantized_decode_quantize_amd import bqd
    from bit_quantized_decode_quantize_amd import decode_stream as DS

    layers = a.layers or 28
    s = DS.QwenW4A8Stream(layers=layers, device=dev, persistent=False)
    c = DS.DecodeChain(s)
    modes = ("producers", "prologue", "fp32")
    logits = {}
    for m in modes:
        c.step(m)
        torch.cuda.synchronize()
        logits[m] = c.output().clone()
    if not all(torch.equal(logits[m], logits["producers"]) for m in modes):
        raise RuntimeError("the chain's modes disagree")
    graph = 0 if a.eager else 1
    timing = {}
    for m in modes:
        ms_m, n_m = time_steps(lambda: c.step(m), a.steps, a.warmup, graph)
        timing[m] = {"ms_per_step": round(ms_m, 5), "launches_per_step": c.launches_per_step(m),
                     "bytes_per_step": c.bytes_per_step(m), "steps": n_m}
        log(f"chain {m}: {timing[m]}")
    ms, n = timing["producers"]["ms_per_step"], timing["producers"]["steps"]
    step_bytes = c.bytes_per_step("producers")
    gbs = step_bytes / (ms * 1e-3) / 1e9

    # Kernel durations in an eager pass of the producers mode: events around
    # the producers and around the int8 GEMVs of gate/up and the lm_head.
    st = torch.cuda.current_stream()
    spans = {"add_rmsnorm_quant": [], "swiglu_quant": [], "gemv": []}
    gemv_bytes = []
    real = dict(add_rmsnorm_quant=bqd.add_rmsnorm_quant, swiglu_quant=bqd.swiglu_quant, gemv_w4a8=bqd.gemv_w4a8)

    def timed(name, key):
        def f(*args, **kw):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            real[name](*args, **kw)
            e1.record(st)
            if key == "gemv":
                N, K = args[0].shape[0], args[0].shape[1] * 8
                if N >= 37888:
                    spans[key].append((e0, e1))
                    gemv_bytes.append(DS.gemv_bytes_q8(N, K, args[2] is not None))
            else:
                spans[key].append((e0, e1))
        return f
    try:
        bqd.add_rmsnorm_quant = timed("add_rmsnorm_quant", "add_rmsnorm_quant")
        bqd.swiglu_quant = timed("swiglu_quant", "swiglu_quant")
        bqd.gemv_w4a8 = timed("gemv_w4a8", "gemv")
        for _ in range(max(1, a.steps // 5)):
            c.step("producers")
    finally:
        bqd.add_rmsnorm_quant, bqd.swiglu_quant, bqd.gemv_w4a8 = (
            real["add_rmsnorm_quant"], real["swiglu_quant"], real["gemv_w4a8"])
    torch.cuda.synchronize()
    avg = {k: sum(e0.elapsed_time(e1) for e0, e1 in v) * 1e3 / len(v) for k, v in spans.items()}
    avg_bytes = sum(gemv_bytes) / len(gemv_bytes)
    out = base_line(a, gbs, ms, n, {
        "workload": f"qwen2-7b-shaped {layers}-layer decode chain: residual add + RMSNorm + quant -> QKV, "
                    "O (synthetic attention output), residual add + RMSNorm + quant -> gate/up, "
                    "SwiGLU + quant -> down, final RMSNorm + quant -> int4 lm_head (producers write int8 codes)",
        "launch": "per-kernel, one HIP graph per token" if graph else "per-kernel",
        "layers": layers, "launches_per_step": c.launches_per_step("producers"), "bytes_per_step": step_bytes})
    out["tok_per_s"] = round(1e3 / ms, 2)
    out["modes"] = timing
    out["producer_us"] = {k: round(avg[k], 2) for k in ("add_rmsnorm_quant", "swiglu_quant")}
    out["roofline"] = roofline(avg_bytes / (avg["gemv"] * 1e-6) / 1e9,
                               "k_gemv_w4a8 on int8 codes (gate/up and lm_head, producers mode)", avg["gemv"],
                               avg_bytes)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_chain(c, a.cpu_seconds)
    return out


def cpu_baseline_chain(c, seconds):
    """The C oracle, single-threaded, over layer 0 of the chain (RMSNorm +
    quant, QKV, O with its own quantisation, RMSNorm + quant, gate/up,
    SwiGLU + quant, down), repeated for about ``seconds``."""
    import torch
    import oracle as O
    from bit_quantized_decode_quantize_amd import decode_stream as DS
    lin = c.by_layer[0]
    prep = {}
    for name, d in lin.items():
        W = c.s.fp32_rows(d, torch.arange(d["N"], device=d["wq"].device)).cpu().numpy()
        prep[name] = O.prepare_int4_rowwise(W) + (d["b"].cpu().numpy(),)
    h0 = c.h_in.cpu().numpy()
    g0, g1 = c.gamma[0].cpu().numpy(), c.gamma[1].cpu().numpy()
    xo = lin["o"]["x"].cpu().numpy()
    sample = c.bytes_per_step("producers") // (len(c.by_layer) + 1)

    def once():
        q, s, h1, _ = O.add_rmsnorm_quant(h0, None, g0, DS.RMS_EPS)
        O.gemv_w4a8(*prep["qkv"][:2], prep["qkv"][2], q[0], float(s[0]))
        _, _, _, yo = O.linear_w4a8(*prep["o"][:2], prep["o"][2], xo)
        q, s, h2, _ = O.add_rmsnorm_quant(h1, yo.astype("float32").reshape(1, -1), g1, DS.RMS_EPS)
        _, ygu = O.gemv_w4a8(*prep["gate_up"][:2], prep["gate_up"][2], q[0], float(s[0]))
        qd, sd, _ = O.swiglu_quant(ygu.astype("float32"))
        O.gemv_w4a8(*prep["down"][:2], prep["down"][2], qd, float(sd))
    gbs, reps, el = cpu_loop(once, sample, seconds)
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle", "host": dict(HOST),
            "sample": f"layer 0 of the chain (~{sample} algorithmic bytes, a layer's share of the step), "
                      f"{reps} passes in {el:.1f} s, single-threaded C"}


# VALU instructions per weight of the compiled INT8-X decode loop (k_gemv_int8x:
# one loop iteration decodes 8 weights per lane) and the chip's VALU issue
# rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (a wave64 VALU instruction holds
# its SIMD for 4 cycles).
INT8X_VALU_PER_WEIGHT = 250 / 8
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def run_int8x(a, dev):
    """INT8-X (3,5,8) decode fused into a W8A8 GEMV at two Qwen2-7B linear
    shapes (down [3584, 18944], gate/up [37888, 3584])."""
    import torch
    from bit_quantized_decode_quantize_amd import workloads as WL

    shapes = []
    for N, K in ((3584, 18944), (37888, 3584)):
        w = WL.Int8XPool(N, K, device=dev, rows=a.r)
        ms, n = time_steps(w.step, max(a.steps, 2 * w.copies), a.warmup, w.copies if (not a.eager) else 0)
        valu = N * K * INT8X_VALU_PER_WEIGHT / (ms * 1e-3) / 1e12
        shapes.append({"N": N, "K": K, "us": round(ms * 1e3, 3), "steps": n,
                       "GB/s": round(w.bytes_per_step() / (ms * 1e-3) / 1e9, 1),
                       "bits_per_weight": round(w.bits_per_weight(), 3),
                       "level_shares": [round(c / (N * K), 4) for c in w.counts],
                       "valu_Tops": round(valu, 2), "rotation_copies": w.copies})
        log(f"int8x {N}x{K}: {shapes[-1]}")
        del w
        torch.cuda.empty_cache()
    d = shapes[0]
    out = base_line(a, d["GB/s"], d["us"] * 1e-3, d["steps"], {
        "workload": "INT8-X (3,5,8) encoded int8 weights (level shares 55.5/40.4/4.1 %), decode fused into "
                    "a W8A8 GEMV, down-projection shape [3584, 18944]",
        "launch": "HIP graph" if (not a.eager) else "eager", "N": d["N"], "K": d["K"]}, dtype="int8")
    out["shapes"] = shapes
    out["roofline"] = {"bound": "alu", "achieved": d["valu_Tops"], "peak": round(VALU_PEAK_TOPS, 1),
                       "unit": "T VALU lane-instructions/s", "frac": round(d["valu_Tops"] / VALU_PEAK_TOPS, 4),
                       "traffic": None, "kernel": "k_gemv_int8x (decode + GEMV, one launch)",
                       "avg_launch_us": d["us"], "valu_per_weight": INT8X_VALU_PER_WEIGHT}
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {a.gpus} requested): the path would shard by output "
              "rows (K for the O and down projections, with an int32 all-reduce); --workload shard runs one "
              "GPU's share of a layer at its real shapes", file=sys.stderr)
        sys.exit(2)
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.copy_calibration:
        # One plain device-to-device copy of known size, for scaling the
        # memory counters of a profiled run.
        src = torch.empty(a.copy_calibration << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {src.numel() * 4} bytes read, {dst.numel() * 4} bytes written")
        del src, dst
        torch.cuda.empty_cache()
    out = {"stream": run_stream, "single": run_single, "layer": run_layer, "gemma": run_gemma,
           "verify": run_verify, "chain": run_chain, "int8x": run_int8x, "shard": run_shard}[a.workload](a, dev)
    print(json.dumps(out), flush=True)
    # Tear the device state down before the interpreter exits: every launch
    # done, the workload's buffers and passes dropped, torch's cache empty.
    import gc
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()
    torch.cuda.synchronize()
    log("done")


if __name__ == "__main__":
    main()
