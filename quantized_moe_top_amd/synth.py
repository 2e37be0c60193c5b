"""Seeded synthetic inputs for the W4 MoE layer.

This module only draws and lays out inputs; it holds none of the layer's
arithmetic (no routing, no dequantisation, no GEMM).  Both the HIP path and
the CPU oracle consume what it produces, and nothing else is shared between
them.

Formats produced (the library's input contract):

* activations ``x``: bf16 ``[T, H]`` row-major.
* router: either fp32 logits ``[T, E]`` or a bf16 router weight ``[E, H]``.
* each W4 bank (gate, up: ``N = I, K = H``; down: ``N = H, K = I``):
  ``qweight`` int32 ``[E, N, K/8]`` whose word ``w`` of a row holds the 4-bit
  codes of columns ``8w .. 8w+7``, code ``8w + j`` in bits ``4j .. 4j+3``
  (lowest nibble first); ``scales`` and ``biases`` bf16 ``[E, N, K/G]``, group
  ``g`` covering reduction indices ``[gG, (g+1)G)``; the weight is
  ``q * scale + bias``.

Workloads (sizes and value distributions follow the layer's benchmark
workloads; every tensor comes from one ``torch.Generator`` seeded once per
layer and drawn in a fixed order: gate, up, down banks (codes expert by
expert, then the scale draw), router weight, activations, logits):

=====================  ==========================================================
name                   contents
=====================  ==========================================================
tiny_t16               T=16, H=256, I=128, E=8, top-2, G=32, logits N(0,1),
                       scale U(0.005, 0.02)
prefill_t512           T=512, H=2048, I=512, E=128, top-8, G=64, bf16 router
                       weight N(0, 0.02), scale U(0.002, 0.01)
decode_t1, decode_t8   the same layer shape at T=1 / T=8, logits N(0,1)
imbalanced_t8192       T=8192, logits N(0,1) - 2.2 ln(e+1) (Zipf-like load),
                       experts with e mod 4 == 3 forced to -inf (no tokens)
longctx_t32768         T=32768, router weight on device, 1% of rows x30,
                       four independently seeded layers
=====================  ==========================================================
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

__all__ = [
    "W4Bank", "MoELayer", "WORKLOADS", "make_layer", "make_custom",
    "pack_codes", "decode_logits_pool",
]


@dataclasses.dataclass
class W4Bank:
    qweight: torch.Tensor  # int32 [E, N, K/8]
    scales: torch.Tensor   # bf16  [E, N, K/G]
    biases: torch.Tensor   # bf16  [E, N, K/G]

    def to(self, device) -> "W4Bank":
        return W4Bank(self.qweight.to(device), self.scales.to(device), self.biases.to(device))

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.qweight, self.scales, self.biases))


@dataclasses.dataclass
class MoELayer:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    G: int
    x: torch.Tensor                        # bf16 [T, H]
    logits: Optional[torch.Tensor]         # fp32 [T, E] or None
    router_weight: Optional[torch.Tensor]  # bf16 [E, H] or None
    gate: W4Bank
    up: W4Bank
    down: W4Bank
    seed: int

    def to(self, device) -> "MoELayer":
        return dataclasses.replace(
            self,
            x=self.x.to(device),
            logits=None if self.logits is None else self.logits.to(device),
            router_weight=None if self.router_weight is None else self.router_weight.to(device),
            gate=self.gate.to(device), up=self.up.to(device), down=self.down.to(device),
        )

    @property
    def weight_bytes_per_expert(self) -> int:
        return (self.gate.nbytes + self.up.nbytes + self.down.nbytes) // self.E


WORKLOADS: Dict[str, dict] = {
    "tiny_t16": dict(T=16, H=256, I=128, E=8, k=2, G=32, router="logits",
                     scale=(0.005, 0.02), seed=1),
    "prefill_t512": dict(T=512, H=2048, I=512, E=128, k=8, G=64, router="weight",
                         scale=(0.002, 0.01), seed=2),
    "decode_t1": dict(T=1, H=2048, I=512, E=128, k=8, G=64, router="logits",
                      scale=(0.002, 0.01), seed=3),
    "decode_t8": dict(T=8, H=2048, I=512, E=128, k=8, G=64, router="logits",
                      scale=(0.002, 0.01), seed=3),
    "imbalanced_t8192": dict(T=8192, H=2048, I=512, E=128, k=8, G=64, router="logits",
                             scale=(0.002, 0.01), seed=4, zipf=True, empty_mod4=True),
    "longctx_t32768": dict(T=32768, H=2048, I=512, E=128, k=8, G=64, router="weight",
                           scale=(0.002, 0.01), seed=5, heavy_frac=0.01, heavy_mul=30.0,
                           layers=4),
}


def pack_codes(q: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes ``q`` (uint8 ``[..., K]``, values 0..15) into uint32
    words ``[..., K/8]``, code ``8w+j`` in bits ``4j..4j+3`` of word ``w``."""
    q = np.asarray(q)
    if q.shape[-1] % 8:
        raise ValueError("K must be a multiple of 8")
    if q.size and (q.max() > 15):
        raise ValueError("codes must be in 0..15")
    words = np.zeros(q.shape[:-1] + (q.shape[-1] // 8,), dtype=np.uint32)
    for j in range(8):
        words |= q[..., j::8].astype(np.uint32) << np.uint32(4 * j)
    return words


def _draw_bank(gen: torch.Generator, E: int, N: int, K: int, G: int,
               scale_lo: float, scale_hi: float, codes=None, bias: str = "m8") -> W4Bank:
    words = np.empty((E, N, K // 8), dtype=np.uint32)
    for e in range(E):
        if codes is None:
            q = torch.randint(0, 16, (N, K), generator=gen, dtype=torch.uint8).numpy()
        else:
            q = np.broadcast_to(np.asarray(codes(e, N, K), dtype=np.uint8), (N, K))
        words[e] = pack_codes(q)
    u = torch.rand((E, N, K // G), generator=gen, dtype=torch.float32)
    scales = (scale_lo + (scale_hi - scale_lo) * u).to(torch.bfloat16)
    if bias == "m8":
        # bias = -8 * scale: exact in bf16 (a power-of-two multiple of a bf16 value)
        biases = (-8.0 * scales.float()).to(torch.bfloat16)
    elif bias == "zeropoint":
        # bias = -m * scale with a zero point m ~ U(2, 14) drawn per group
        m = 2.0 + 12.0 * torch.rand((E, N, K // G), generator=gen, dtype=torch.float32)
        biases = (-m * scales.float()).to(torch.bfloat16)
    elif bias == "free":
        # bias drawn independently of the scale: N(0, (4 * mean scale)^2)
        sd = 2.0 * (scale_lo + scale_hi)
        biases = (sd * torch.randn((E, N, K // G), generator=gen, dtype=torch.float32)).to(torch.bfloat16)
    else:
        raise ValueError(bias)
    qweight = torch.from_numpy(words.view(np.int32).copy())
    return W4Bank(qweight, scales, biases)


def make_custom(T: int, H: int, I: int, E: int, k: int, G: int, seed: int, *,
                router: str = "logits", scale=(0.002, 0.01), zipf: bool = False,
                empty_mod4: bool = False, heavy_frac: float = 0.0, heavy_mul: float = 1.0,
                bias: str = "m8", name: Optional[str] = None) -> MoELayer:
    """Draw one layer; ``router`` is ``"logits"`` (fp32 N(0,1) logits given)
    or ``"weight"`` (bf16 router weight N(0, 0.02), logits computed on device).
    ``bias`` picks the per-group bias: ``"m8"`` (-8 * scale, the benchmark
    workloads), ``"zeropoint"`` (-m * scale, m ~ U(2, 14) per group) or
    ``"free"`` (N(0, (4 * mean scale)^2), independent of the scale)."""
    if H % G or I % G or H % 8 or I % 8:
        raise ValueError("H and I must be multiples of G and 8")
    gen = torch.Generator().manual_seed(seed)
    gate = _draw_bank(gen, E, I, H, G, *scale, bias=bias)
    up = _draw_bank(gen, E, I, H, G, *scale, bias=bias)
    down = _draw_bank(gen, E, H, I, G, *scale, bias=bias)
    router_weight = None
    if router == "weight":
        router_weight = (0.02 * torch.randn((E, H), generator=gen)).to(torch.bfloat16)
    x = torch.randn((T, H), generator=gen, dtype=torch.float32)
    if heavy_frac > 0 and T > 0:
        n_heavy = int(round(heavy_frac * T))
        rows = torch.randperm(T, generator=gen)[:n_heavy]
        x[rows] *= heavy_mul
    x = x.to(torch.bfloat16)
    logits = None
    if router == "logits":
        logits = torch.randn((T, E), generator=gen, dtype=torch.float32)
        if zipf:
            rank = torch.arange(1, E + 1, dtype=torch.float64)
            logits = logits + (2.0 * (-1.1) * torch.log(rank)).to(torch.float32)
        if empty_mod4:
            logits[:, 3::4] = float("-inf")
    elif router != "weight":
        raise ValueError(router)
    return MoELayer(name or f"custom_t{T}", T, H, I, E, k, G, x, logits, router_weight,
                    gate, up, down, seed)


def make_layer(name: str, layer_index: int = 0) -> MoELayer:
    """Draw one of the named workloads (``layer_index`` selects one of the
    independently seeded layers of ``longctx_t32768``)."""
    cfg = dict(WORKLOADS[name])
    layers = cfg.pop("layers", 1)
    if not 0 <= layer_index < layers:
        raise ValueError(f"{name} has {layers} layer(s)")
    seed = cfg.pop("seed") + layer_index
    return make_custom(seed=seed, name=name, **cfg)


def decode_logits_pool(T: int, E: int, n: int, seed: int) -> torch.Tensor:
    """``n`` independent fp32 N(0,1) logit sets ``[n, T, E]`` for rotating the
    touched experts between timed decode steps."""
    gen = torch.Generator().manual_seed(seed)
    return torch.randn((n, T, E), generator=gen, dtype=torch.float32)


# ------------------------------------------------ decode attention inputs --
@dataclasses.dataclass
class AttnCase:
    """One decode-attention step: one query token per sequence against a
    block-paged key/value cache (``kcache`` bf16 ``[NB, Hkv, BLK, D]``,
    position-major; ``vcache`` bf16 ``[NB, Hkv, D, BLK]``, element-major;
    ``table`` int32 ``[B, MB]`` maps block i of sequence b to a physical
    block; ``lens`` int32 ``[B]``)."""
    name: str
    q: torch.Tensor
    kcache: torch.Tensor
    vcache: torch.Tensor
    table: torch.Tensor
    lens: torch.Tensor
    block: int

    def to(self, device) -> "AttnCase":
        return dataclasses.replace(self, q=self.q.to(device), kcache=self.kcache.to(device),
                                   vcache=self.vcache.to(device), table=self.table.to(device),
                                   lens=self.lens.to(device))


def make_attention(lens, Hq: int = 32, Hkv: int = 4, D: int = 128, block: int = 64,
                   seed: int = 90, name: str = "attn") -> AttnCase:
    """Seeded decode-attention inputs: q, K and V bf16 N(0, 1); each sequence
    gets ceil(len / block) blocks (at least one), and the physical blocks of
    all sequences are one seeded permutation, so consecutive positions of a
    sequence sit in scattered blocks.  Draw order: permutation, q, K, V (V
    drawn position-major, stored element-major)."""
    gen = torch.Generator().manual_seed(seed)
    lens = [int(n) for n in lens]
    B = len(lens)
    nblk = [max(1, -(-n // block)) for n in lens]
    NB, MB = sum(nblk), max(nblk)
    perm = torch.randperm(NB, generator=gen)
    table = torch.zeros((B, MB), dtype=torch.int32)
    pos = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[pos:pos + n].to(torch.int32)
        pos += n
    q = torch.randn(B, Hq, D, generator=gen).to(torch.bfloat16)
    kc = torch.randn(NB, Hkv, block, D, generator=gen).to(torch.bfloat16)
    vc = torch.randn(NB, Hkv, block, D, generator=gen).to(torch.bfloat16).transpose(2, 3).contiguous()
    return AttnCase(name, q, kc, vc, table, torch.tensor(lens, dtype=torch.int32), block)


# Decode-attention workloads: the context lengths the pages quote their
# decode gains at (32K and 128K), one sequence and a batch of eight.
ATTN_WORKLOADS = {
    "attn_decode_32k": dict(lens=[32768], seed=91),
    "attn_decode_128k": dict(lens=[131072], seed=92),
    "attn_decode_b8_32k": dict(lens=[32768] * 8, seed=93),
}


def make_attention_workload(name: str) -> AttnCase:
    return make_attention(name=name, **ATTN_WORKLOADS[name])
