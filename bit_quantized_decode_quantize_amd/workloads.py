"""Resident benchmark workloads besides the 28-layer stream, run through the C ABI.

Each class builds its tensors on the GPU from the seeded generator, keeps
them resident, and exposes ``step()`` (one unit of work, enqueued on the
current stream), ``bytes_per_step()`` (the algorithmic bytes of that unit)
and, where the unit is not a whole launch, ``launches_per_step``.

Weights that fit the 256 MB Infinity Cache are replicated into a rotation
pool of distinct device copies (same content, different addresses) that
together exceed 1 GB; consecutive steps walk the pool, so every step streams
its weights from HBM, as a decode step over a full model does.

* ``SingleGemvPool``: one Q-projection GEMV [3584, 3584] (per-row INT4,
  fused per-token activation quantisation, 1 % of x scaled by 20).
* ``LayerPool``: one Qwen2-7B-shaped decoder layer (fused QKV, O, fused
  gate/up, down), per-linear launches or the persistent pass.
* ``GemmaG32Stream``: 35 Gemma-shaped layers of group-32 INT4 linears with
  fp16 activations plus the lm_head [262144, 1536], int8-expanded (W8A16) or
  packed 6-bit (section 3 of "在香橙派上跑 Gemma4：vLLM 适配昇腾 310B 的内核开发实录").
* ``VerifyPool``: the M-token verify GEMM over [18944, 3584] or
  [3584, 18944] (section 5 of the same page).
* ``ShardLayerPool``: one GPU's share of the Qwen2-7B-shaped layer under
  8-way tensor parallelism (output rows of QKV and gate/up, a K slice of O
  and down with int32 partial accumulators).
* ``Int8XPool``: INT8-X (3,5,8) encoded int8 weights ("定長無損 INT8 壓縮與
  Triton 融合解碼") at a Qwen2-7B linear's shape, codes drawn with the page's
  level shares, through the decode-fused W8A8 GEMV.
"""
from __future__ import annotations

from typing import Dict, List

import torch

from . import bqd
from . import inputs as I
from .decode_stream import _qwen_part_shapes, algorithmic_bytes_linear, layer_biases, layer_inputs, linear_weight_fp32

POOL_BYTES = 1 << 30


def _copies(nbytes: int, minimum: int) -> int:
    return max(minimum, -(-POOL_BYTES // nbytes))


def bytes_group32_linear(N: int, K: int, bias: bool, x_bytes: int = 2) -> int:
    """Group-32 W4A8 linear: packed weights N*K/2, fp16 scales 2*N*K/32,
    bias 4N, x read once, y 4N."""
    return N * K // 2 + 2 * N * (K // 32) + (4 * N if bias else 0) + K * x_bytes + 4 * N


def bytes_w8a16(N: int, K: int) -> int:
    """W8A16 GEMV: int8 codes N*K, fp16 scales 2*N*K/32, fp16 x 2K, y 4N."""
    return N * K + 2 * N * (K // 32) + 2 * K + 4 * N


def bytes_q6k(N: int, K: int) -> int:
    """Packed 6-bit GEMV: 210 bytes per 256 weights, fp16 x 2K, y 4N."""
    return N * K * 210 // 256 + 2 * K + 4 * N


def bytes_verify(M: int, N: int, K: int, bias: bool = True) -> int:
    """Verify GEMM: packed weights N*K/2, scales 4N, bias 4N, codes M*K,
    token scales 4M, y 4*M*N."""
    return N * K // 2 + 4 * N + (4 * N if bias else 0) + M * K + 4 * M + 4 * M * N


class SingleGemvPool:
    """The single Q-projection linear: W [3584, 3584] ~N(0, 0.02^2) per-row
    INT4, x fp32 [3584] ~N(0, 1) with 1 % of entries x20, bias ~N(0, 0.01^2).
    One step = one fused linear (quantise x, GEMV) on the next pool copy."""

    def __init__(self, seed: int = 0, device="cuda", N: int = 3584, K: int = 3584, r: int = 0,
                 lanes_per_row: int = 0):
        self.device = torch.device(device)
        self.r, self.lanes_per_row = r, lanes_per_row
        d = I.single_gemv_inputs(seed, self.device, K=K, N=N)
        wq, sw = bqd.quantize_weights_int4_rowwise(d["W"])
        del d["W"]
        self.N, self.K = N, K
        self.copies = _copies(wq.numel() * 4, 160)
        self.wq = wq.unsqueeze(0).repeat(self.copies, 1, 1)
        self.sw = sw.unsqueeze(0).repeat(self.copies, 1)
        self.b = d["b"].unsqueeze(0).repeat(self.copies, 1)
        self.x = d["x"]
        self.y = torch.empty(N, dtype=torch.float32, device=self.device)
        self.i = 0
        self.launches_per_step = 1
        torch.cuda.synchronize(self.device)

    def step(self, stream=None) -> None:
        c = self.i % self.copies
        self.i += 1
        bqd.linear_w4a8(self.wq[c], self.sw[c], self.b[c], self.x, y=self.y, r=self.r,
                        lanes_per_row=self.lanes_per_row, stream=stream)

    def bytes_per_step(self) -> int:
        return algorithmic_bytes_linear(self.N, self.K, True)

    def weight_bytes(self) -> int:
        return self.N * self.K // 2


class LayerPool:
    """One Qwen2-7B-shaped decoder layer (the four fused linears of layer 0
    of the 28-layer stream), replicated into >= 9 copies.  One step = one
    layer: four fused launches (``layer_w4a8_forward``), or, persistent,
    one launch of the pass runs every copy in turn (``copies`` layer steps),
    each linear reading the previous linear's output."""

    def __init__(self, seed: int = 0, device="cuda", persistent: bool = False):
        self.device = torch.device(device)
        prefix = "qwen/L0"
        biases = layer_biases(prefix, seed, self.device)
        inputs = layer_inputs(prefix, seed, self.device)
        base = []
        for name, N, K in I.qwen_layer_linears():
            W = linear_weight_fp32(prefix, name, seed, self.device)
            wq, sw = bqd.quantize_weights_int4_rowwise(W)
            del W
            base.append(dict(name=name, N=N, K=K, wq=wq, sw=sw, b=biases[name], x=inputs[name]))
        layer_bytes = sum(d["N"] * d["K"] // 2 for d in base)
        self.copies = _copies(layer_bytes, 9)
        self.layers: List[List[Dict]] = []
        self.plans: List[bqd.LayerPlan] = []
        for c in range(self.copies):
            lin = []
            for d in base:
                e = dict(d)
                if c:
                    e.update(wq=d["wq"].clone(), sw=d["sw"].clone(), b=d["b"].clone())
                e["y"] = torch.empty(d["N"], dtype=torch.float32, device=self.device)
                lin.append(e)
            self.layers.append(lin)
            self.plans.append(bqd.LayerPlan([bqd.make_linear(e["wq"], e["sw"], e["b"]) for e in lin],
                                            [e["x"] for e in lin], [e["y"] for e in lin]))
        self.persistent = persistent
        self.pass_ = None
        if persistent:
            # chained as a decoder chains them: each linear reads the first K
            # values of the previous linear's output (the first one its own x)
            flat = [e for lin in self.layers for e in lin]
            xs = [flat[0]["x"]] + [flat[i - 1]["y"][:e["K"]] for i, e in enumerate(flat) if i > 0]
            self.pass_ = bqd.DecodePass([bqd.make_linear(e["wq"], e["sw"], e["b"]) for e in flat],
                                        xs, [e["y"] for e in flat], self.device)
        self.i = 0
        self.launches_per_step = 1.0 / self.copies if persistent else 4
        self.steps_per_call = self.copies if persistent else 1
        torch.cuda.synchronize(self.device)

    def step(self, stream=None) -> None:
        """Persistent: one launch = ``copies`` layers; otherwise one layer."""
        if self.pass_ is not None:
            self.pass_.run(stream)
        else:
            self.plans[self.i % self.copies].run(stream)
            self.i += 1

    def bytes_per_step(self) -> int:
        return sum(algorithmic_bytes_linear(e["N"], e["K"], True) for e in self.layers[0])

    def weight_bytes(self) -> int:
        return sum(e["N"] * e["K"] // 2 for e in self.layers[0])


def shard_row_index(name: str, rank: int, G: int, device) -> torch.Tensor:
    """Rows of a fused linear that rank ``rank`` of ``G`` holds when the
    output rows are split: the same share of each fused part (q, k, v; gate,
    up), so every GPU holds whole heads and matching gate and up rows."""
    parts, _ = _qwen_part_shapes()[name]
    idx, off = [], 0
    for _, n in parts:
        if n % G:
            raise ValueError(f"{name}: {n} rows do not split {G} ways")
        idx.append(torch.arange(off + rank * (n // G), off + (rank + 1) * (n // G)))
        off += n
    return torch.cat(idx).to(device)


def bytes_partial_gemv(N: int, K: int) -> int:
    """A K-slice GEMV on int8 codes with int32 partials: packed weights N*K/2,
    scales 4N, codes K, s^x 4, y 4N and the int32 partials 4N (the entry
    point writes y as well; the partials are what the all-reduce sums)."""
    return N * K // 2 + 4 * N + K + 4 + 4 * N + 4 * N


class ShardLayerPool:
    """One GPU's share of the Qwen2-7B-shaped decoder layer (layer 0 of the
    stream) under G-way tensor parallelism, at its real shapes:

    * QKV and gate/up split by output rows ([576, 3584] and [4736, 3584] at
      G = 8): x is replicated and every GPU quantises it bit-identically in
      the fused linear, so no reduction is needed;
    * O and down split along K ([3584, 448] and [3584, 2368]): each GPU
      computes exact int32 partial accumulators over its K slice on the
      activation's codes (s^x being the all-reduced maximum, the codes are
      the full activation's), an int32 all-reduce of [N] would sum them
      exactly, and the per-row epilogue (scale, bias) runs once after it.

    Replicated into >= 1 GB of copies; one step = the share's four launches."""

    def __init__(self, seed: int = 0, device="cuda", G: int = 8, rank: int = 0):
        self.device = torch.device(device)
        self.G, self.rank = G, rank
        prefix = "qwen/L0"
        biases = layer_biases(prefix, seed, self.device)
        inputs = layer_inputs(prefix, seed, self.device)
        base = []
        for name, N, K in I.qwen_layer_linears():
            W = linear_weight_fp32(prefix, name, seed, self.device)
            wq, sw = bqd.quantize_weights_int4_rowwise(W)
            del W
            if name in ("qkv", "gate_up"):
                rows = shard_row_index(name, rank, G, self.device)
                base.append(dict(name=name, kind="rows", N=rows.numel(), K=K, wq=wq[rows].contiguous(),
                                 sw=sw[rows].contiguous(), b=biases[name][rows].contiguous(), x=inputs[name]))
            else:
                if K % (32 * G):
                    raise ValueError(f"{name}: K = {K} does not split {G} ways into whole 32-value groups")
                ks = K // G
                k0 = rank * ks
                qx, sx = bqd.quantize_act(inputs[name])
                base.append(dict(name=name, kind="k", N=N, K=ks, k0=k0,
                                 wq=wq[:, k0 // 8:(k0 + ks) // 8].contiguous(), sw=sw, b=None,
                                 qx=qx[k0:k0 + ks].contiguous(), sx=sx))
            del wq
        share = sum(d["N"] * d["K"] // 2 for d in base)
        self.copies = _copies(share, 9)
        self.layers: List[List[Dict]] = []
        for c in range(self.copies):
            lin = []
            for d in base:
                e = dict(d)
                if c:
                    e.update(wq=d["wq"].clone(), sw=d["sw"].clone())
                    if d["b"] is not None:
                        e["b"] = d["b"].clone()
                e["y"] = torch.empty(d["N"], dtype=torch.float32, device=self.device)
                if d["kind"] == "k":
                    e["acc"] = torch.empty(d["N"], dtype=torch.int32, device=self.device)
                lin.append(e)
            self.layers.append(lin)
        self.i = 0
        self.launches_per_step = 4
        torch.cuda.synchronize(self.device)

    @staticmethod
    def run_linear(e, stream=None) -> None:
        if e["kind"] == "rows":
            bqd.linear_w4a8(e["wq"], e["sw"], e["b"], e["x"], y=e["y"], stream=stream)
        else:
            bqd.gemv_w4a8(e["wq"], e["sw"], None, e["qx"], e["sx"], y=e["y"], acc=e["acc"], stream=stream)

    def step(self, stream=None) -> None:
        for e in self.layers[self.i % self.copies]:
            self.run_linear(e, stream)
        self.i += 1

    @staticmethod
    def linear_bytes(e) -> int:
        if e["kind"] == "rows":
            return algorithmic_bytes_linear(e["N"], e["K"], True)
        return bytes_partial_gemv(e["N"], e["K"])

    def bytes_per_step(self) -> int:
        return sum(self.linear_bytes(e) for e in self.layers[0])

    def weight_bytes(self) -> int:
        return sum(e["N"] * e["K"] // 2 for e in self.layers[0])


class GemmaG32Stream:
    """35 Gemma-shaped layers (fused QKV [2048, 1536], O [1536, 2048], fused
    gate/up [12288, 1536], down [1536, 6144]) of group-32 INT4 weights with
    fp16 scales and fp16 activations, no bias, plus the lm_head [262144, 1536]
    as int8 codes in [-32, 31] with fp16 group-32 scales (W8A16).  One step =
    one token: 140 fused group-32 linears + the W8A16 lm_head, one launch each.
    Weights total 1.1 GB, so every step streams from HBM."""

    def __init__(self, layers: int = 35, seed: int = 0, device="cuda", r: int = 0, lanes_per_row: int = 0,
                 head: str = "w8a16"):
        if head not in ("w8a16", "q6k"):
            raise ValueError(f"unknown lm_head form {head}")
        self.device = torch.device(device)
        self.r, self.lanes_per_row = r, lanes_per_row
        self.head = head
        self.linears: List[Dict] = []
        for l in range(layers):
            prefix = f"gemma/L{l}"
            for name, N, K in I.gemma_layer_linears():
                W = I.normal(f"{prefix}/{name}/W", (N, K), 0.02, seed, self.device)
                wq, s16 = bqd.quantize_weights_int4_group32(W)
                del W
                x = I.linear_input(prefix, name, K, seed, self.device, torch.float16)
                y = torch.empty(N, dtype=torch.float32, device=self.device)
                self.linears.append(dict(layer=l, name=name, N=N, K=K, wq=wq, s16=s16, x=x, y=y))
        N, K = I.GEMMA["vocab"], I.GEMMA["hidden"]
        W = I.normal("gemma/lm_head/W", (N, K), 0.02, seed, self.device)
        self.w8, self.w8s = bqd.quantize_weights_int8_group32(W)
        self.q6k = bqd.quantize_weights_q6k(W)
        del W
        self.head_x = I.normal("gemma/lm_head/x", K, 1.0, seed, self.device, torch.float16)
        self.head_y = torch.empty(N, dtype=torch.float32, device=self.device)
        self.head_NK = (N, K)
        self.launches_per_step = len(self.linears) + 1
        torch.cuda.synchronize(self.device)

    def step(self, stream=None) -> None:
        for d in self.linears:
            bqd.linear_w4a8_group32(d["wq"], d["s16"], None, d["x"], y=d["y"], r=self.r,
                                    lanes_per_row=self.lanes_per_row, stream=stream)
        self.run_head(stream)

    def run_head(self, stream=None) -> None:
        if self.head == "q6k":
            self.lm_head_q6k(stream)
        else:
            self.lm_head(stream)

    def make_pass(self, chained: bool = True) -> "bqd.DecodePass":
        """The 140 group-32 linears as one persistent pass.  chained: linear
        i reads the first K_i values of linear i-1's output (fp32, through
        the pass's exchange; linear 0 reads its activation widened to fp32),
        outputs in ``.outputs``; otherwise each linear reads its own fp16
        activation and writes the stream's outputs."""
        lins = [bqd.make_linear(d["wq"], d["s16"], None) for d in self.linears]
        if chained:
            ys = [torch.empty(d["N"], dtype=torch.float32, device=self.device) for d in self.linears]
            x0 = self.linears[0]["x"].float()
            xs = [x0] + [ys[i - 1][:d["K"]] for i, d in enumerate(self.linears) if i > 0]
        else:
            ys = [d["y"] for d in self.linears]
            xs = [d["x"] for d in self.linears]
        p = bqd.DecodePass(lins, xs, ys, self.device)
        p.outputs = ys
        p.inputs = xs
        return p

    def pass_bytes(self, chained: bool = True) -> int:
        """Algorithmic bytes of the pass's linears (fp32 activations when
        chained, fp16 otherwise) plus the lm_head."""
        xb = 4 if chained else 2
        return sum(bytes_group32_linear(d["N"], d["K"], False, xb) for d in self.linears) + self.head_bytes()

    def lm_head(self, stream=None) -> None:
        """The int8-expanded lm_head (W8A16, fp16 group-32 scales)."""
        bqd.gemv_w8a16_group32(self.w8, self.w8s, self.head_x, y=self.head_y, stream=stream)

    def lm_head_q6k(self, stream=None) -> None:
        """The packed 6-bit lm_head, decoded in registers."""
        bqd.gemv_q6k_f16(self.q6k, self.head_x, y=self.head_y, stream=stream)

    def head_bytes(self, head=None) -> int:
        return bytes_q6k(*self.head_NK) if (head or self.head) == "q6k" else bytes_w8a16(*self.head_NK)

    def bytes_per_step(self) -> int:
        return sum(bytes_group32_linear(d["N"], d["K"], False) for d in self.linears) + self.head_bytes()

    def weight_bytes(self) -> int:
        N, K = self.head_NK
        head = N * K * 210 // 256 if self.head == "q6k" else N * K + 2 * N * (K // 32)
        return sum(d["N"] * d["K"] // 2 + 2 * d["N"] * (d["K"] // 32) for d in self.linears) + head


class VerifyPool:
    """M-token verify over one per-row INT4 weight ([18944, 3584] gate-shaped
    or [3584, 18944] down-shaped), W ~N(0, 0.02^2), bias ~N(0, 0.01^2),
    X fp32 [M, K] ~N(0, 1) quantised per token once (outside the step).
    One step = one verify GEMM on the next of >= 30 pool copies."""

    def __init__(self, N: int, K: int, M: int, seed: int = 0, device="cuda", impl: int = 0):
        self.device = torch.device(device)
        self.N, self.K, self.M, self.impl = N, K, M, impl
        W = I.normal(f"verify/{N}x{K}/W", (N, K), 0.02, seed, self.device)
        wq, sw = bqd.quantize_weights_int4_rowwise(W)
        del W
        b = I.normal(f"verify/{N}x{K}/b", N, 0.01, seed, self.device)
        X = I.normal(f"verify/{N}x{K}/X", (M, K), 1.0, seed, self.device)
        self.qx, self.sx = bqd.quantize_act(X)
        self.copies = _copies(wq.numel() * 4, 30)
        self.wq = wq.unsqueeze(0).repeat(self.copies, 1, 1)
        self.sw = sw.unsqueeze(0).repeat(self.copies, 1)
        self.b = b.unsqueeze(0).repeat(self.copies, 1)
        self.y = torch.empty(M, N, dtype=torch.float32, device=self.device)
        self.i = 0
        self.launches_per_step = 1
        torch.cuda.synchronize(self.device)

    def step(self, stream=None) -> None:
        c = self.i % self.copies
        self.i += 1
        bqd.gemm_w4a8_verify(self.wq[c], self.sw[c], self.b[c], self.qx, self.sx, y=self.y,
                             impl=self.impl, stream=stream)

    def bytes_per_step(self) -> int:
        return bytes_verify(self.M, self.N, self.K)

    def int_ops_per_step(self) -> int:
        return 2 * self.N * self.K * self.M

    def weight_bytes(self) -> int:
        return self.N * self.K // 2


class Int8XPool:
    """INT8-X encoded int8 weights [N, K] (codes with the page's level shares
    55.5 / 40.4 / 4.1 %), int8 x ~ uniform, per-tensor scales; one step = one
    decode-fused W8A8 GEMV on the next of >= 16 pool copies."""

    def __init__(self, N: int, K: int, seed: int = 0, device="cuda", rows: int = 0):
        self.device = torch.device(device)
        self.N, self.K, self.rows = N, K, rows
        q = I.int8_codes_by_band(f"int8x/{N}x{K}/q", (N, K), seed=seed)
        base = bqd.int8x_encode(q, 0.0042, device=self.device)
        self.counts = base.counts
        self.copies = _copies(base.nbytes(), 16)
        self.pool = [base] + [bqd.Int8XWeights({k: v.clone() for k, v in base.arrays.items()}, base.sizes,
                                               base.counts, N, K, base.sw) for _ in range(self.copies - 1)]
        self.qx = I.uniform_int(f"int8x/{N}x{K}/x", K, -127, 127, seed, self.device, torch.int8)
        self.sx = torch.tensor([0.0173], device=self.device)
        self.y = torch.empty(N, dtype=torch.float32, device=self.device)
        self.i = 0
        self.launches_per_step = 1
        torch.cuda.synchronize(self.device)

    def step(self, stream=None) -> None:
        w = self.pool[self.i % self.copies]
        self.i += 1
        bqd.gemv_int8x(w, self.qx, self.sx, y=self.y, rows=self.rows, stream=stream)

    def bytes_per_step(self) -> int:
        """Encoded payload (bitmaps and streams, unpadded) + block sums + x + y."""
        w = self.pool[0]
        blocks = self.N * self.K // bqd.BQD_INT8X_BLOCK
        return (w.payload_bits() + 7) // 8 + 8 * (blocks + 1) + self.K + 4 * self.N

    def bits_per_weight(self) -> float:
        return self.pool[0].payload_bits() / (self.N * self.K)
