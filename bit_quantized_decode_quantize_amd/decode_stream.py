"""Resident W4A8 decode weight streams, built on the GPU and run through the C ABI.

``QwenW4A8Stream`` holds the Qwen2-7B-shaped decoder (28 layers, hidden
3584, KV 512, intermediate 18944, vocab 152064) as per-row INT4 weights in
HBM: per layer the four linears after load-time fusion (q/k/v rows
concatenated, gate/up rows concatenated, as section 3.1 of "在香橙派上跑
Gemma4：vLLM 适配昇腾 310B 的内核开发实录" does), plus an int4 per-row
lm_head.  One ``step()`` is one token's pass over the whole weight stream:
for every linear, in decoder order on one stream, the activation is
quantised and the GEMV runs, in a single launch per linear.

Weights come from the seeded generator (fp32 ~N(0, 0.02^2)), quantised on
the device by the library's load-time kernel; each linear's activation is a
resident synthetic vector (N(0, 1), or silu(g)*u for the down projection),
standing in for the output of the operators between GEMVs that are outside
this path (norms, attention, residuals).
"""
from __future__ import annotations

import os
from typing import Dict, List, Optional, Tuple

import torch

from . import bqd
from . import inputs as I

QKV_PARTS = (("q", "hidden"), ("k", "kv_dim"), ("v", "kv_dim"))
GATE_UP_PARTS = (("gate", "inter"), ("up", "inter"))


def _qwen_part_shapes():
    h, kv, i = I.QWEN["hidden"], I.QWEN["kv_dim"], I.QWEN["inter"]
    size = dict(hidden=h, kv_dim=kv, inter=i)
    return {
        "qkv": ([(p, size[s]) for p, s in QKV_PARTS], h),
        "o": ([("o", h)], h),
        "gate_up": ([(p, size[s]) for p, s in GATE_UP_PARTS], h),
        "down": ([("down", h)], i),
    }


def linear_weight_fp32(prefix: str, name: str, seed: int, device) -> torch.Tensor:
    """fp32 weight of one fused linear: its parts generated separately and
    their rows concatenated (load-time fusion)."""
    parts, K = _qwen_part_shapes()[name]
    return torch.cat([I.normal(f"{prefix}/{p}/W", (n, K), 0.02, seed, device) for p, n in parts])


def layer_biases(prefix: str, seed: int, device) -> Dict[str, torch.Tensor]:
    """fp32 biases ~N(0, 0.01^2) of one layer's four fused linears, drawn in
    one stream and split in row order (q, k, v | o | gate, up | down)."""
    sizes = [(name, N) for name, N, _ in I.qwen_layer_linears()]
    allb = I.normal(f"{prefix}/biases", sum(n for _, n in sizes), 0.01, seed, device)
    return dict(zip([nm for nm, _ in sizes], torch.split(allb, [n for _, n in sizes])))


def layer_inputs(prefix: str, seed: int, device) -> Dict[str, torch.Tensor]:
    """Activations of one layer's four linears: N(0, 1) for QKV, O and gate/up
    (one stream, split), silu(g)*u for the down projection."""
    lin = I.qwen_layer_linears()
    ks = [K for name, _, K in lin if name != "down"]
    xs = torch.split(I.normal(f"{prefix}/x", sum(ks), 1.0, seed, device), ks)
    out = dict(zip([name for name, _, _ in lin if name != "down"], [x.contiguous() for x in xs]))
    out["down"] = I.swiglu_like(f"{prefix}/down/x", dict((n, k) for n, _, k in lin)["down"], seed, device)
    return out


def load_cache(path: str, meta: Dict[str, str], device) -> Optional[Dict[str, torch.Tensor]]:
    """Tensors of a stream cache written by ``QwenW4A8Stream.save``, copied
    to ``device``, or None when ``path`` is missing or holds another stream.
    safetensors stores raw tensors only: nothing in the file is executed."""
    from safetensors import safe_open
    if not os.path.exists(path):
        return None
    with safe_open(path, framework="pt", device="cpu") as f:
        if f.metadata() != meta:
            return None
        return {k: f.get_tensor(k).to(device) for k in f.keys()}


def algorithmic_bytes_linear(N: int, K: int, bias: bool, x_bytes: int = 4) -> int:
    """Bytes one fused decode linear must move: packed weights N*K/2, fp32
    scales 4N, bias 4N, the activation x (read once), the output y 4N."""
    return N * K // 2 + 4 * N + (4 * N if bias else 0) + K * x_bytes + 4 * N


CACHE_FORMAT = "qwen-w4a8-stream/1"


class QwenW4A8Stream:
    """``cache``: path of a safetensors file holding a stream built earlier
    with the same layers, seed and head (``save``); when it matches, every
    tensor is copied from it instead of being generated and quantised, so
    the process launches none of the generator's or quantiser's kernels."""

    def __init__(self, layers: int = 28, seed: int = 0, device="cuda", lm_head: bool = True,
                 r: int = 0, lanes_per_row: int = 0, persistent: bool = True, cache: Optional[str] = None):
        self.device = torch.device(device)
        self.layers = layers
        self.seed = seed
        self.lm_head = lm_head
        self.linears: List[Dict] = []       # every linear in step order
        self.plans: List[bqd.LayerPlan] = []
        self.cached = load_cache(cache, self.cache_meta(), self.device) if cache else None
        c = self.cached
        for l in range(layers):
            prefix = f"qwen/L{l}"
            descs, xs, ys = [], [], []
            if c is None:
                biases = layer_biases(prefix, seed, self.device)
                inputs = layer_inputs(prefix, seed, self.device)
            for name, N, K in I.qwen_layer_linears():
                i = len(self.linears)
                if c is not None:
                    wq, sw, b, x = c[f"{i}.wq"], c[f"{i}.sw"], c.get(f"{i}.b"), c[f"{i}.x"]
                else:
                    W = linear_weight_fp32(prefix, name, seed, self.device)
                    assert W.shape == (N, K)
                    wq, sw = bqd.quantize_weights_int4_rowwise(W)
                    del W
                    b = biases[name]
                    x = inputs[name]
                y = torch.empty(N, dtype=torch.float32, device=self.device)
                d = dict(layer=l, name=name, N=N, K=K, wq=wq, sw=sw, b=b, x=x, y=y, prefix=prefix)
                self.linears.append(d)
                descs.append(bqd.make_linear(wq, sw, b, r, lanes_per_row))
                xs.append(x)
                ys.append(y)
            self.plans.append(bqd.LayerPlan(descs, xs, ys))
        if lm_head:
            N, K = I.QWEN["vocab"], I.QWEN["hidden"]
            i = len(self.linears)
            if c is not None:
                wq, sw, x = c[f"{i}.wq"], c[f"{i}.sw"], c[f"{i}.x"]
            else:
                W = I.normal("qwen/lm_head/W", (N, K), 0.02, seed, self.device)
                wq, sw = bqd.quantize_weights_int4_rowwise(W)
                del W
                x = I.normal("qwen/lm_head/x", K, 1.0, seed, self.device)
            y = torch.empty(N, dtype=torch.float32, device=self.device)
            self.linears.append(dict(layer=layers, name="lm_head", N=N, K=K, wq=wq, sw=sw, b=None,
                                     x=x, y=y, prefix="qwen/lm_head"))
            self.plans.append(bqd.LayerPlan([bqd.make_linear(wq, sw, None, r, lanes_per_row)],
                                            [x], [y]))
        self.persistent = persistent
        self.pass_ = None
        if persistent:
            self.pass_ = bqd.DecodePass(
                [bqd.make_linear(d["wq"], d["sw"], d["b"]) for d in self.linears],
                [d["x"] for d in self.linears], [d["y"] for d in self.linears], self.device)
        torch.cuda.synchronize(self.device)

    def step(self, stream=None) -> None:
        """One token: every linear in order.  Persistent: one launch for the
        whole pass; otherwise one fused launch per linear."""
        if self.pass_ is not None:
            self.pass_.run(stream)
        else:
            for p in self.plans:
                p.run(stream)

    def chained_pass(self) -> "bqd.DecodePass":
        """The same linears chained as a decoder chains them, in one pass:
        linear i reads the first K_i values of linear i-1's output (through
        output buffers of its own; ``.outputs``), linear 0 the stream's
        activation.  Same algorithmic bytes as a step of the stream; each
        linear waits for the previous one's rows (the decoder's dependency)."""
        ys = [torch.empty(d["N"], dtype=torch.float32, device=self.device) for d in self.linears]
        xs = [self.linears[0]["x"]] + [ys[i - 1][:d["K"]] for i, d in enumerate(self.linears) if i > 0]
        p = bqd.DecodePass([bqd.make_linear(d["wq"], d["sw"], d["b"]) for d in self.linears], xs, ys, self.device)
        p.outputs = ys
        return p

    def link_floor_pass(self, size: int = 64) -> "bqd.DecodePass":
        """As many linears as the stream, each [size, size] and chained like
        ``chained_pass``: the dependency between consecutive linears (store,
        poll, staging, a few rows) with next to no weight traffic."""
        n = len(self.linears)
        wq, sw, x0 = self._link_floor_tensors(size)
        ys = [torch.empty(size, dtype=torch.float32, device=self.device) for _ in range(n)]
        lins = [bqd.make_linear(wq[i * size:(i + 1) * size], sw[i * size:(i + 1) * size], None) for i in range(n)]
        p = bqd.DecodePass(lins, [x0] + ys[:-1], ys, self.device)
        p.outputs = ys
        return p

    def cut_pass(self, rows: int = 64) -> "bqd.DecodePass":
        """The same linears cut to their first ``rows`` rows (views of the
        stream's weights) with the stream's own activations, in one pass;
        outputs in ``.outputs``."""
        ys = [torch.empty(rows, dtype=torch.float32, device=self.device) for _ in self.linears]
        lins = [bqd.make_linear(d["wq"][:rows], d["sw"][:rows], None if d["b"] is None else d["b"][:rows])
                for d in self.linears]
        p = bqd.DecodePass(lins, [d["x"] for d in self.linears], ys, self.device)
        p.outputs = ys
        return p

    def _link_floor_tensors(self, size: int):
        key = f"linkfloor{size}"
        if self.cached is not None and f"{key}.wq" in self.cached:
            return self.cached[f"{key}.wq"], self.cached[f"{key}.sw"], self.cached[f"{key}.x"]
        W = I.normal("qwen/linkfloor/W", (len(self.linears) * size, size), 0.02, self.seed, self.device)
        wq, sw = bqd.quantize_weights_int4_rowwise(W)
        del W
        return wq, sw, I.normal("qwen/linkfloor/x", size, 1.0, self.seed, self.device)

    def cache_meta(self) -> Dict[str, str]:
        return {"format": CACHE_FORMAT, "layers": str(self.layers), "seed": str(self.seed),
                "lm_head": str(int(self.lm_head))}

    def save(self, path: str, link_floor_sizes=(64,)) -> None:
        """Write every tensor the stream generated (weights, scales, biases,
        activations, and the link-floor linears of ``link_floor_sizes``)
        to ``path`` (safetensors, written to a temporary name and renamed)."""
        from safetensors.torch import save_file
        t = {}
        for i, d in enumerate(self.linears):
            t[f"{i}.wq"], t[f"{i}.sw"], t[f"{i}.x"] = d["wq"], d["sw"], d["x"]
            if d["b"] is not None:
                t[f"{i}.b"] = d["b"]
        for size in link_floor_sizes:
            t[f"linkfloor{size}.wq"], t[f"linkfloor{size}.sw"], t[f"linkfloor{size}.x"] = \
                self._link_floor_tensors(size)
        t = {k: v.detach().contiguous().cpu() for k, v in t.items()}
        tmp = f"{path}.tmp{os.getpid()}"
        save_file(t, tmp, metadata=self.cache_meta())
        os.replace(tmp, path)

    def bytes_per_step(self) -> int:
        return sum(algorithmic_bytes_linear(d["N"], d["K"], d["b"] is not None) for d in self.linears)

    def weight_bytes(self) -> int:
        return sum(d["N"] * d["K"] // 2 for d in self.linears)

    def fp32_rows(self, d: Dict, rows: torch.Tensor) -> torch.Tensor:
        """Regenerate the fp32 weight rows ``rows`` of linear ``d`` (same seed)."""
        if d["name"] == "lm_head":
            W = I.normal("qwen/lm_head/W", (d["N"], d["K"]), 0.02, self.seed, self.device)
        else:
            W = linear_weight_fp32(d["prefix"], d["name"], self.seed, self.device)
        out = W[rows.to(self.device)].clone()
        del W
        return out


RMS_EPS = 1e-6


def producer_bytes_rmsnorm(K: int, residual: bool, codes: bool) -> int:
    """Residual add + RMSNorm producer: reads h (+ delta) and gamma, writes
    h + delta, then int8 codes and s^x (or the fp32 values)."""
    return 4 * K * (3 if residual else 2) + (K + 4 if codes else 4 * K)


def producer_bytes_swiglu(I_: int, codes: bool) -> int:
    """SwiGLU producer: reads gate and up (8I), writes codes and s^x (or fp32 h)."""
    return 8 * I_ + (I_ + 4 if codes else 4 * I_)


def gemv_bytes_q8(N: int, K: int, bias: bool) -> int:
    """GEMV on int8 codes: packed weights, scales, bias, codes + s^x, y."""
    return N * K // 2 + 4 * N + (4 * N if bias else 0) + K + 4 + 4 * N


class DecodeChain:
    """The stream's linears wired into a decoder's data flow, with the
    producers of the activations ([Orin] "后续还能继续优化什么", items 1-2):

        per layer:  h1 = h + y_down(prev); x = RMSNorm(h1)  -> QKV
                    (attention is outside the path: the O projection reads a
                     synthetic attention output and quantises it itself)
                    h2 = h1 + y_O;         x = RMSNorm(h2)  -> gate/up
                    x = silu(gate) * up                     -> down
        final:      x = RMSNorm(h + y_down)                 -> lm_head

    Three ways to run it, with the same codes from the same fp32 values and
    hence outputs identical bit for bit:
      "producers": each producer writes int8 codes + s^x and the linears are
        int8 GEMVs (``add_rmsnorm_quant`` / ``swiglu_quant``, ``gemv_w4a8``);
      "fp32": the producers write fp32 and each linear quantises in its own
        prologue (``linear_w4a8``);
      "prologue": the residual add + RMSNorm + quantisation run inside the
        prologue of the linear that consumes them (``linear_rmsnorm_w4a8``),
        SwiGLU as in "producers" (its elementwise work is too large to
        repeat in every workgroup of the down projection).
    The residual stream starts from the same h_in every step."""

    def __init__(self, stream: "QwenW4A8Stream", seed: int = 0):
        self.s = stream
        dev = stream.device
        K, I_ = I.QWEN["hidden"], I.QWEN["inter"]
        self.K, self.I = K, I_
        L = stream.layers
        self.h_in = I.normal("qwen/chain/h0", (1, K), 1.0, seed, dev)
        g = 1.0 + I.normal("qwen/chain/gamma", (2 * L + 1, K), 0.1, seed, dev)
        self.gamma = [g[i].contiguous() for i in range(2 * L + 1)]
        self.h = torch.empty(1, K, device=dev)
        self.h2 = torch.empty(1, K, device=dev)  # "prologue": h + delta alternates between the two
        self.q_h = torch.empty(1, K, dtype=torch.int8, device=dev)
        self.s_h = torch.empty(1, device=dev)
        self.q_i = torch.empty(1, I_, dtype=torch.int8, device=dev)
        self.s_i = torch.empty(1, device=dev)
        self.y_h = torch.empty(1, K, device=dev)
        self.y_i = torch.empty(1, I_, device=dev)
        self.by_layer = [dict((d["name"], d) for d in stream.linears if d["layer"] == l) for l in range(L)]
        self.head = stream.linears[-1] if stream.linears[-1]["name"] == "lm_head" else None
        torch.cuda.synchronize(dev)

    def _norm(self, fused, src, delta, gamma, stream):
        if fused:
            bqd.add_rmsnorm_quant(src, gamma, RMS_EPS, delta=delta, h_out=self.h, qx=self.q_h, sx=self.s_h,
                                  stream=stream)
        else:
            bqd.add_rmsnorm_quant(src, gamma, RMS_EPS, delta=delta, h_out=self.h, y_out=self.y_h,
                                  quantize=False, stream=stream)

    def _linear_h(self, fused, d, stream):
        if fused:
            bqd.gemv_w4a8(d["wq"], d["sw"], d["b"], self.q_h.view(-1), self.s_h, y=d["y"], stream=stream)
        else:
            bqd.linear_w4a8(d["wq"], d["sw"], d["b"], self.y_h.view(-1), y=d["y"], stream=stream)

    def step(self, mode: str = "producers", stream=None) -> None:
        if mode == "prologue":
            return self._step_prologue(stream)
        if mode not in ("producers", "fp32"):
            raise ValueError(f"unknown chain mode {mode}")
        fused = mode == "producers"
        delta = None
        for l, lin in enumerate(self.by_layer):
            self._norm(fused, self.h_in if l == 0 else self.h, delta, self.gamma[2 * l], stream)
            self._linear_h(fused, lin["qkv"], stream)
            o = lin["o"]
            bqd.linear_w4a8(o["wq"], o["sw"], o["b"], o["x"], y=o["y"], stream=stream)
            self._norm(fused, self.h, o["y"].view(1, -1), self.gamma[2 * l + 1], stream)
            self._linear_h(fused, lin["gate_up"], stream)
            gu, dn = lin["gate_up"]["y"].view(1, -1), lin["down"]
            if fused:
                bqd.swiglu_quant(gu, h_out=self.y_i, qx=self.q_i, sx=self.s_i, stream=stream)
                bqd.gemv_w4a8(dn["wq"], dn["sw"], dn["b"], self.q_i.view(-1), self.s_i, y=dn["y"], stream=stream)
            else:
                bqd.swiglu_quant(gu, h_out=self.y_i, quantize=False, stream=stream)
                bqd.linear_w4a8(dn["wq"], dn["sw"], dn["b"], self.y_i.view(-1), y=dn["y"], stream=stream)
            delta = dn["y"].view(1, -1)
        if self.head is not None:
            self._norm(fused, self.h, delta, self.gamma[-1], stream)
            self._linear_h(fused, self.head, stream)

    def _step_prologue(self, stream=None) -> None:
        bufs = (self.h, self.h2)
        src, delta, k = self.h_in, None, 0

        def rms_linear(d, gamma):
            nonlocal src, k
            dst = bufs[k]
            bqd.linear_rmsnorm_w4a8(d["wq"], d["sw"], d["b"], src.view(-1), gamma, RMS_EPS,
                                    delta=None if delta is None else delta.view(-1), h_out=dst.view(-1),
                                    y=d["y"], stream=stream)
            src, k = dst, 1 - k

        for l, lin in enumerate(self.by_layer):
            rms_linear(lin["qkv"], self.gamma[2 * l])
            o = lin["o"]
            bqd.linear_w4a8(o["wq"], o["sw"], o["b"], o["x"], y=o["y"], stream=stream)
            delta = o["y"]
            rms_linear(lin["gate_up"], self.gamma[2 * l + 1])
            dn = lin["down"]
            bqd.swiglu_quant(lin["gate_up"]["y"].view(1, -1), h_out=self.y_i, qx=self.q_i, sx=self.s_i,
                             stream=stream)
            bqd.gemv_w4a8(dn["wq"], dn["sw"], dn["b"], self.q_i.view(-1), self.s_i, y=dn["y"], stream=stream)
            delta = dn["y"]
        if self.head is not None:
            rms_linear(self.head, self.gamma[-1])

    def output(self) -> torch.Tensor:
        return (self.head or self.by_layer[-1]["down"])["y"]

    def launches_per_step(self, mode: str = "producers") -> int:
        # per layer: QKV, O, gate/up and down, plus two RMSNorm producers
        # (not in "prologue") and SwiGLU (two kernels with codes, one for fp32)
        per_layer = {"producers": 8, "fp32": 7, "prologue": 6}[mode]
        head = 1 if mode == "prologue" else 2
        return per_layer * len(self.by_layer) + (head if self.head is not None else 0)

    def bytes_per_step(self, mode: str = "producers") -> int:
        K, I_ = self.K, self.I
        if mode == "prologue":
            return self._bytes_prologue()
        fused = mode == "producers"
        tot = 0
        for l, lin in enumerate(self.by_layer):
            tot += producer_bytes_rmsnorm(K, l > 0, fused) + producer_bytes_rmsnorm(K, True, fused)
            tot += producer_bytes_swiglu(I_, fused)
            o = lin["o"]
            tot += algorithmic_bytes_linear(o["N"], o["K"], True)
            for name in ("qkv", "gate_up", "down"):
                d = lin[name]
                tot += gemv_bytes_q8(d["N"], d["K"], d["b"] is not None) if fused else \
                    algorithmic_bytes_linear(d["N"], d["K"], d["b"] is not None)
        if self.head is not None:
            d = self.head
            tot += producer_bytes_rmsnorm(K, True, fused)
            tot += gemv_bytes_q8(d["N"], d["K"], False) if fused else algorithmic_bytes_linear(d["N"], d["K"], False)
        return tot

    def _bytes_prologue(self) -> int:
        """RMSNorm in the consumer's prologue: the linear reads h, delta and
        gamma (12K, 8K without delta) and writes h + delta (4K) instead of
        reading K bytes of codes; SwiGLU as with producers."""
        K, I_ = self.K, self.I
        tot = 0
        for l, lin in enumerate(self.by_layer):
            for name, with_delta in (("qkv", l > 0), ("gate_up", True)):
                d = lin[name]
                tot += gemv_bytes_q8(d["N"], d["K"], True) - (K + 4) + 4 * K * (3 if with_delta else 2) + 4 * K
            o = lin["o"]
            tot += algorithmic_bytes_linear(o["N"], o["K"], True)
            tot += producer_bytes_swiglu(I_, True) + gemv_bytes_q8(lin["down"]["N"], lin["down"]["K"], True)
        if self.head is not None:
            d = self.head
            tot += gemv_bytes_q8(d["N"], d["K"], False) - (K + 4) + 16 * K
        return tot
