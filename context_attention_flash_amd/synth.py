"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and rounds them to bfloat16; it holds none of
the attention arithmetic (no positions, masks, softmax or merge).  Both the HIP
path and the fp64 oracle consume the arrays it returns, so they see identical
values.

Workloads (shapes follow the long-context training cases the ring-attention
pages describe; every tensor is drawn over the *global* sequence in global
token order, as [B, N, H, d]):

* ``tiny_fp32``   -- batch 1, 2 heads, d 64, N 512, D 4, fp32 N(0,1)*0.1,
                     non-causal, basic layout (the 0.1 scale follows the numpy
                     demonstration on the ai360xpert "Ring Attention" page,
                     "Show Me the Code").
* ``basic_s4096`` -- basic causal, N 32768, D 8, rank 7, 32 heads, d 128, bf16.
* ``zigzag``      -- zigzag causal, N 131072, D 8, rank 3, GQA 32/8, bf16.
* ``llama3``      -- packed 65536 tokens, llama3 layout, rank 5, GQA 32/8, bf16,
                     documents with lognormal lengths (median 2048, sigma 1.0,
                     clipped to [64, 16384]).
* ``basic_s8192`` -- basic causal fwd+bwd, N 65536, D 8, rank 7, 32 heads, bf16.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Layout codes; the same integers are used by the C ABI.
BASIC, ZIGZAG, STRIPE, VARLEN_RING, LLAMA3, VARLEN_ZIGZAG, VARLEN_STRIPE = 0, 1, 2, 3, 4, 5, 6
LAYOUT_NAMES = {BASIC: "basic", ZIGZAG: "zigzag", STRIPE: "stripe",
                VARLEN_RING: "varlen_ring", LLAMA3: "llama3",
                VARLEN_ZIGZAG: "varlen_zigzag", VARLEN_STRIPE: "varlen_stripe"}
# layouts over packed documents (batch 1, cu_seqlens required)
VARLEN_LAYOUTS = (VARLEN_RING, LLAMA3, VARLEN_ZIGZAG, VARLEN_STRIPE)


def doc_multiple(layout: int, world: int) -> int:
    """Document lengths a packed layout accepts must be multiples of this."""
    return {VARLEN_RING: world, VARLEN_STRIPE: world, VARLEN_ZIGZAG: 2 * world}.get(layout, 1)


# Document boundaries of the packed llama3 workload.  They were produced once by
# ``lognormal_cu_seqlens(65536, 2048, 1.0, 64, 16384, np.random.default_rng(2004))``
# with numpy 2.2 and are kept literally so that the workload does not depend on
# the numpy version.
LLAMA3_CU_SEQLENS = [0, 2579, 6771, 10364, 13336, 14508, 15162, 25106, 27500,
                     30198, 31283, 47667, 54130, 56256, 57381, 65536]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    seqlen: int            # global N (total packed tokens for varlen layouts)
    world: int             # D
    rank: int              # r (the rank whose share is computed)
    causal: bool
    layout: int
    dtype: str             # "bf16" or "f32"
    seed: int
    value_scale: float = 1.0
    cu_seqlens: Optional[tuple] = None
    with_grad: bool = False
    window: tuple = (-1, -1)   # sliding window (left, right); -1 = unbounded side

    @property
    def shard(self) -> int:
        return self.seqlen // self.world

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 2, 2, 64, 512, 4, 0, False, BASIC, "f32",
                          seed=1001, value_scale=0.1),
    "basic_s4096": Workload("basic_s4096", 1, 32, 32, 128, 32768, 8, 7, True, BASIC,
                            "bf16", seed=1002),
    "zigzag": Workload("zigzag", 1, 32, 8, 128, 131072, 8, 3, True, ZIGZAG, "bf16",
                       seed=1003),
    "llama3": Workload("llama3", 1, 32, 8, 128, 65536, 8, 5, True, LLAMA3, "bf16",
                       seed=1004, cu_seqlens=tuple(LLAMA3_CU_SEQLENS)),
    "basic_s8192": Workload("basic_s8192", 1, 32, 32, 128, 65536, 8, 7, True, BASIC,
                            "bf16", seed=1005, with_grad=True),
}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs are finite by construction.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    rounded = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(bf16_round_bits(x))


def lognormal_cu_seqlens(total: int, median: float, sigma: float, lo: int, hi: int,
                         rng: np.random.Generator) -> list:
    """Draw document lengths one by one (lognormal, rounded, clipped to [lo, hi])
    until they cover ``total`` tokens; the last document is cut so that the
    lengths sum to ``total`` exactly.  Returns cu_seqlens (prefix sums, leading 0)."""
    cu = [0]
    while cu[-1] < total:
        length = int(np.clip(np.rint(rng.lognormal(np.log(median), sigma)), lo, hi))
        cu.append(min(cu[-1] + length, total))
    return cu


def random_cu_seqlens(total: int, n_docs: int, rng: np.random.Generator,
                      multiple: int = 1) -> list:
    """Random document split of ``total`` tokens into ``n_docs`` non-empty
    documents whose lengths are multiples of ``multiple``."""
    units = total // multiple
    assert units * multiple == total and n_docs <= units
    cuts = np.sort(rng.choice(np.arange(1, units), size=n_docs - 1, replace=False))
    return [0] + [int(c) * multiple for c in cuts] + [total]


def draw_global(w: Workload, rng: Optional[np.random.Generator] = None) -> dict:
    """Draw Q, K, V (and dO when the workload has a backward pass) over the
    global sequence, in global token order, as [B, N, H, d] float32 arrays
    holding exactly representable bf16 values for bf16 workloads."""
    if rng is None:
        rng = np.random.default_rng(w.seed)
    shp_q = (w.batch, w.seqlen, w.heads_q, w.head_dim)
    shp_kv = (w.batch, w.seqlen, w.heads_kv, w.head_dim)
    out = {}
    for name, shp in (("q", shp_q), ("k", shp_kv), ("v", shp_kv)):
        out[name] = rng.standard_normal(shp, dtype=np.float32) * np.float32(w.value_scale)
    if w.with_grad:
        out["dout"] = rng.standard_normal(shp_q, dtype=np.float32)
    if w.dtype == "bf16":
        for name in list(out):
            out[name] = quantize_bf16(out[name])
    return out
