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

from typing import Dict, List, Tuple

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


def algorithmic_bytes_linear(N: int, K: int, bias: bool, x_bytes: int = 4) -> int:
    """Bytes one fused decode linear must move: packed weights N*K/2, fp32
    scales 4N, bias 4N, the activation x (read once), the output y 4N."""
    return N * K // 2 + 4 * N + (4 * N if bias else 0) + K * x_bytes + 4 * N


class QwenW4A8Stream:
    def __init__(self, layers: int = 28, seed: int = 0, device="cuda", lm_head: bool = True,
                 r: int = 0, lanes_per_row: int = 0, persistent: bool = True):
        self.device = torch.device(device)
        self.layers = layers
        self.seed = seed
        self.linears: List[Dict] = []       # every linear in step order
        self.plans: List[bqd.LayerPlan] = []
        for l in range(layers):
            prefix = f"qwen/L{l}"
            descs, xs, ys = [], [], []
            biases = layer_biases(prefix, seed, self.device)
            inputs = layer_inputs(prefix, seed, self.device)
            for name, N, K in I.qwen_layer_linears():
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
