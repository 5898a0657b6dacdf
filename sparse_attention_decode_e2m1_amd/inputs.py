"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds none of the method's arithmetic: it only draws random
numbers (host ``torch.Generator``), rounds activations to bf16 with torch's
cast, and encodes the sliding-window rows to FP8 E4M3 with torch's cast and a
per-tensor scale (the window cache is an input of the path, written upstream).

Seed of every tensor: ``1_000_000*c + 1000*b + 10*layer + t`` where c is the
workload index, b the sequence, layer the layer's place in the group and t the
tensor kind (0 main KV, 1 index keys, 2 q, 3 indexer q, 4 indexer weights,
5 window rows, 6 salient direction).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch

T_KV, T_IKEY, T_Q, T_QI, T_W, T_SWA, T_SAL = range(7)
FULL, REINDEX, REUSE = 0, 1, 2
SWA = 3  # a layer that attends to its own window only (no global entries)
MODE_NAMES = ("FULL", "REINDEX", "REUSE", "SWA")


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: head/latent/indexer sizes are those of the
    pages' model family (16 query heads over a 576-channel latent = 512 + 64
    rope, an indexer of 4 heads x 128, a 128-token window)."""
    name: str
    index: int              # c in the seed formula
    B: int                  # sequences
    N: int                  # context length (cache rows per sequence)
    K: int                  # Top-K
    modes: tuple            # layer modes of the group, in order
    T: int = 1              # query tokens per sequence (prefill chunk when > 1)
    P: int = 0              # candidate pool size kept by the first FULL layer
    H: int = 16
    D: int = 576
    DV: int = 512
    HI: int = 4
    DI: int = 128
    W: int = 128
    salient: bool = False

    @property
    def ctx0(self) -> int:
        """Rows cached before the query tokens of the step."""
        return self.N - self.T

    @property
    def sm_scale(self) -> float:
        return float(torch.tensor(1.0 / (self.D ** 0.5), dtype=torch.float32))


C1 = Workload("C1_full_4k", 0, B=1, N=4096, K=256, modes=(FULL,))
C2 = Workload("C2_full_b16_64k", 1, B=16, N=65536, K=2048, modes=(FULL,))
C3 = Workload("C3_group_b4_256k", 2, B=4, N=262144, K=2048,
              modes=(FULL, REINDEX, REUSE, REUSE))
C4 = Workload("C4_pool_1m", 3, B=1, N=1048576, K=2048,
              modes=(FULL, REINDEX, REINDEX), P=16384, salient=True)
C5 = Workload("C5_prefill_4k_on_128k", 4, B=1, N=135168, K=2048,
              modes=(FULL,), T=4096)


def forty_layer_modes() -> tuple:
    """The static layer plan of the pages' 40-layer model (helmcode.com/
    deepseek-v41-flash, section "03 · CSA2": 4 Full, 4 Reindex and 30 Reuse
    attention layers plus 2 window-only layers, the window-only ones first).
    The pages give the counts, not the order of the rest; read here as four
    groups of a Full layer, then its Reindex layer, then Reuse layers (8, 8,
    7, 7), each group over its own caches."""
    modes = [SWA, SWA]
    for n in (8, 8, 7, 7):
        modes += [FULL, REINDEX] + [REUSE] * n
    return tuple(modes)


# The 40-layer decode step at contexts 4K .. 1M (one sequence, Top-K 2048).
F1 = tuple(Workload(f"F1_40layer_{tag}", 5 + j, B=1, N=n, K=2048, modes=forty_layer_modes())
           for j, (tag, n) in enumerate((("4k", 4096), ("16k", 16384), ("64k", 65536),
                                         ("256k", 262144), ("1m", 1048576))))
WORKLOADS = {w.name: w for w in (C1, C2, C3, C4, C5) + F1}


def group_of_layers(modes) -> list:
    """Cache group of each layer: each Full layer starts a group with its
    own caches; layers before the first Full layer belong to group 0."""
    g, out = -1, []
    for m in modes:
        if m == FULL:
            g += 1
        out.append(max(g, 0))
    return out


def seed(c: int, b: int, layer: int, t: int) -> int:
    return 1_000_000 * c + 1000 * b + 10 * layer + t


def gen(s: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(s)
    return g


def randn(shape, s: int) -> torch.Tensor:
    return torch.randn(*shape, generator=gen(s), dtype=torch.float32)


def rand(shape, s: int) -> torch.Tensor:
    return torch.rand(*shape, generator=gen(s), dtype=torch.float32)


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def fp8_rows(x: torch.Tensor):
    """E4M3 bytes and the fp32 per-tensor scale amax/448 (torch's cast)."""
    amax = x.abs().max().to(torch.float32)
    scale = (amax / 448.0) if float(amax) > 0 else torch.tensor(1.0)
    b = (x / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return b.contiguous(), float(scale)


def rope_cos_sin(positions, rope_dim: int, base: float = 10000.0) -> torch.Tensor:
    """Rotary angles of the standard form (upstream of the path; the pages
    give no rotary parameters): pair i of a row at position p turns by
    p * base**(-2i/rope_dim).  Returns fp32 [len(positions)][rope_dim/2][2]
    (cos, sin), evaluated in float64 and rounded once."""
    pos = torch.as_tensor(positions, dtype=torch.float64).reshape(-1, 1)
    i = torch.arange(rope_dim // 2, dtype=torch.float64).reshape(1, -1)
    ang = pos * torch.pow(torch.tensor(base, dtype=torch.float64), -2.0 * i / rope_dim)
    return torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).to(torch.float32).contiguous()


def salient_direction(w: Workload, b: int) -> torch.Tensor:
    u = randn((w.DI,), seed(w.index, b, 0, T_SAL))
    return u / u.norm()


def salient_rows(w: Workload, b: int) -> torch.Tensor:
    """A random 1% of positions carry the salient direction."""
    g = gen(seed(w.index, b, 1, T_SAL))
    n = max(1, round(0.01 * w.N))
    return torch.randperm(w.N, generator=g)[:n]


@dataclass
class SeqCache:
    kv: torch.Tensor        # [N][D] fp32 (rows ctx0.. are the new tokens)
    ikey: torch.Tensor      # [N][DI] fp32


@dataclass
class LayerInputs:
    q: torch.Tensor         # [T][H][D] bf16
    q_idx: torch.Tensor     # [T][HI][DI] bf16
    w_idx: torch.Tensor     # [T][HI] fp32
    swa: torch.Tensor       # [S][D] uint8 (E4M3)
    swa_scale: float
    swa_pos0: int           # position of window row 0


def seq_cache(w: Workload, b: int) -> SeqCache:
    """Main KV and index keys of one sequence, N(0,1) fp32.  For a prefill
    chunk the new rows are bf16 activations (rounded here)."""
    kv = randn((w.N, w.D), seed(w.index, b, 0, T_KV))
    ik = randn((w.N, w.DI), seed(w.index, b, 0, T_IKEY))
    if w.salient:
        u = salient_direction(w, b)
        ik[salient_rows(w, b)] += 8.0 * u
    if w.T > 1:
        kv[w.ctx0:] = kv[w.ctx0:].to(torch.bfloat16).float()
        ik[w.ctx0:] = ik[w.ctx0:].to(torch.bfloat16).float()
    return SeqCache(kv, ik)


def layer_inputs(w: Workload, b: int, layer: int) -> LayerInputs:
    q = to_bf16(randn((w.T, w.H, w.D), seed(w.index, b, layer, T_Q)))
    qi = randn((w.T, w.HI, w.DI), seed(w.index, b, layer, T_QI))
    if w.salient:
        qi += 4.0 * salient_direction(w, b)
    qi = to_bf16(qi)
    wi = rand((w.T, w.HI), seed(w.index, b, layer, T_W))
    S = w.W - 1 + w.T
    swa_src = randn((S, w.D), seed(w.index, b, layer, T_SWA))
    swa, sc = fp8_rows(swa_src)
    return LayerInputs(q, qi, wi, swa, sc, w.N - S)


def small(name: str, index: int, B: int, N: int, K: int, modes, T: int = 1,
          P: int = 0, W: int = 128, salient: bool = False, H: int = 16,
          D: int = 576, DV: int = 512, HI: int = 4, DI: int = 128) -> Workload:
    """A reduced workload with the same structure (for tests)."""
    return Workload(name, index, B=B, N=N, K=K, modes=tuple(modes), T=T, P=P,
                    W=W, salient=salient, H=H, D=D, DV=DV, HI=HI, DI=DI)
