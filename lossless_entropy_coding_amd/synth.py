"""Seeded synthetic BF16 workloads (inputs only; no codec arithmetic here).

The pages measure their codec on real checkpoints that are not available
here (a 27.8B-weight BF16 checkpoint of 1,199 tensors on the
Qwen3.8-27B-BF16-NVLC-Lossless card, metrics table; Gemma 2 9B on the
BigSmall card).  These generators stand in for them with the same shapes and
value statistics: normally distributed weights rounded to BF16 with
round-to-nearest-even, per-row or per-tensor scales, outliers and exact
zeros, and FP32 vectors kept verbatim.

Every generator is deterministic for its seed.  ``device`` selects where the
random numbers are drawn ("cpu" default; "cuda" is much faster for the big
workloads, but draws a different, equally seeded stream).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass
class Item:
    name: str
    kind: str                 # "bf16" or "raw"
    tensor: torch.Tensor      # bfloat16 (bf16) or any dtype (raw, kept verbatim)


@dataclass
class Workload:
    name: str
    items: list = field(default_factory=list)
    chunk_weights: int = 65536
    lanes: int = 64
    stream_lanes: int = 0     # lanes per word stream (0: one stream per chunk)
    m_s: int = 12             # precision of the (sign, exponent) table
    m_f: int = 10             # precision of the fraction tables (layout 2: of the h tables, 16 - m_s)
    layout: int = 1           # record layout: 2 codes s and f >> 4 with one renormalisation per weight

    @property
    def n_bf16(self) -> int:
        return sum(i.tensor.numel() for i in self.items if i.kind == "bf16")

    @property
    def raw_bytes(self) -> int:
        return sum(i.tensor.numel() * i.tensor.element_size() for i in self.items if i.kind == "raw")


def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def cfg1(device: str = "cpu") -> Workload:
    """1024x1024 BF16, N(0, 0.02) (0.02 read as the standard deviation), seed 0;
    64 KiB-output chunks (32768 weights) with 32 lanes each."""
    g = _gen(0, device)
    t = (torch.randn(1024, 1024, generator=g, device=device) * 0.02).to(torch.bfloat16)
    return Workload("cfg1_1024x1024_N0.02", [Item("w", "bf16", t)], chunk_weights=32768, lanes=32)


def cfg2(device: str = "cpu", lanes: int = 64) -> Workload:
    """4096x4096 BF16: row scale s_r = exp(log 0.02 + 0.5 z_r); x = z * s_r;
    one U(0,1) draw u per element: u < 0.001 -> x*50 (outlier),
    0.001 <= u < 0.011 -> +0.0 (exact zero); seed 0; 256 KiB chunks."""
    g = _gen(0, device)
    s = torch.exp(math.log(0.02) + 0.5 * torch.randn(4096, 1, generator=g, device=device))
    x = torch.randn(4096, 4096, generator=g, device=device) * s
    u = torch.rand(4096, 4096, generator=g, device=device)
    x = torch.where(u < 0.001, x * 50.0, x)
    x = torch.where((u >= 0.001) & (u < 0.011), torch.zeros_like(x), x)
    return Workload("cfg2_4096x4096_lognormal_rows_outliers_zeros", [Item("w", "bf16", x.to(torch.bfloat16))],
                    chunk_weights=131072, lanes=lanes)


GEMMA2_9B_LAYER = [
    ("q_proj", (3584, 4096)), ("k_proj", (3584, 2048)), ("v_proj", (3584, 2048)), ("o_proj", (4096, 3584)),
    ("gate_proj", (3584, 14336)), ("up_proj", (3584, 14336)), ("down_proj", (14336, 3584)),
]


def cfg3(device: str = "cpu", chunk_weights: int = 65536, lanes: int = 128) -> Workload:
    """One Gemma-2-9B-shaped decoder layer: seven BF16 matrices N(0, 0.02)
    (seeds 0..6) and four FP32 norm vectors of 3584 (1 + 0.02 z, seeds 7..10)
    carried verbatim as the residual."""
    items = []
    for i, (name, shape) in enumerate(GEMMA2_9B_LAYER):
        g = _gen(i, device)
        items.append(Item(name, "bf16", (torch.randn(*shape, generator=g, device=device) * 0.02).to(torch.bfloat16)))
    for j in range(4):
        g = _gen(7 + j, device)
        v = 1.0 + 0.02 * torch.randn(3584, generator=g, device=device, dtype=torch.float32)
        items.append(Item(f"norm{j}", "raw", v))
    return Workload("cfg3_gemma2_9b_layer", items, chunk_weights=chunk_weights, lanes=lanes)


def cfg4(device: str = "cpu", chunk_weights: int = 65536, lanes: int = 128, rows: int = 256000) -> Workload:
    """256000x3584 embedding-shaped BF16 tensor; row std = exp(U(log 0.005,
    log 0.05)); generated in row blocks of 8192 from one seeded stream."""
    g = _gen(0, device)
    cols = 3584
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device=device)
    lo, hi = math.log(0.005), math.log(0.05)
    for r0 in range(0, rows, 8192):
        r1 = min(rows, r0 + 8192)
        std = torch.exp(lo + (hi - lo) * torch.rand(r1 - r0, 1, generator=g, device=device))
        out[r0:r1] = (torch.randn(r1 - r0, cols, generator=g, device=device) * std).to(torch.bfloat16)
    return Workload("cfg4_embedding_256000x3584", [Item("embed", "bf16", out)],
                    chunk_weights=chunk_weights, lanes=lanes)


def cfg5_layout(hidden: int = 5120, inter: int = 17408, kv: int = 1024, layers: int = 84, tail_vectors: int = 23):
    """Tensor list (name, shape) of the ~27.7B-weight synthetic checkpoint:
    per layer gate/up (hidden x inter), down (inter x hidden), q/o (hidden x
    hidden), k/v (kv x hidden) and seven vectors of hidden; plus trailing
    vectors.  84 layers give 588 matrices + 611 vectors = 1,199 tensors."""
    out = []
    for L in range(layers):
        out += [(f"l{L}.gate", (hidden, inter)), (f"l{L}.up", (hidden, inter)), (f"l{L}.down", (inter, hidden)),
                (f"l{L}.q", (hidden, hidden)), (f"l{L}.o", (hidden, hidden)),
                (f"l{L}.k", (kv, hidden)), (f"l{L}.v", (kv, hidden))]
        out += [(f"l{L}.vec{j}", (hidden,)) for j in range(7)]
    out += [(f"tail.vec{j}", (hidden,)) for j in range(tail_vectors)]
    return out


def cfg5_tensor(index: int, shape, device: str = "cpu") -> torch.Tensor:
    """Tensor `index` of the synthetic checkpoint: std = exp(U(log 0.003,
    log 0.1)) drawn first from a generator seeded with the tensor index."""
    g = _gen(index, device)
    lo, hi = math.log(0.003), math.log(0.1)
    std = math.exp(lo + (hi - lo) * float(torch.rand(1, generator=g, device=device).item()))
    return (torch.randn(*shape, generator=g, device=device) * std).to(torch.bfloat16)


def cfg5_layer(layer: int, device: str = "cpu", chunk_weights: int = 65536, lanes: int = 128,
               layout=None) -> Workload:
    """The 14 tensors of one layer of the synthetic checkpoint (or the tail
    vectors when layer == number of layers)."""
    layout = layout or cfg5_layout()
    per_layer = 14
    n_layers = (len(layout) - 23) // per_layer
    if layer < n_layers:
        idx = range(layer * per_layer, (layer + 1) * per_layer)
    else:
        idx = range(n_layers * per_layer, len(layout))
    items = [Item(layout[i][0], "bf16", cfg5_tensor(i, layout[i][1], device)) for i in idx]
    return Workload(f"cfg5_layer{layer}", items, chunk_weights=chunk_weights, lanes=lanes)


def special_words() -> torch.Tensor:
    """Every one of the 65,536 BF16 bit patterns (zeros, subnormals, infs, all
    NaN payloads) as an int16-viewed bfloat16 tensor."""
    w = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    return w.view(torch.bfloat16)


def as_words(t: torch.Tensor) -> torch.Tensor:
    """The raw 16-bit pattern of a bfloat16 tensor (int16 view, flattened)."""
    return t.contiguous().reshape(-1).view(torch.int16)


CONFIGS = {"1": cfg1, "2": cfg2, "3": cfg3, "4": cfg4}
