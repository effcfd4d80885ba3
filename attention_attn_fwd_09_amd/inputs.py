"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the attention arithmetic, so both the HIP path and the fp64
oracle can consume its tensors without sharing any computation.

Recipe (the pages use no public dataset; every tensor is synthetic):

* one host ``torch.Generator`` per tensor, seeded ``1000 * config + t`` with
  t = 0 (Q), 1 (K), 2 (V), 3 (dO), 4 (padding lengths), 5 (block layout);
* Q, K, V, dO are i.i.d. N(0, 1) drawn in float32 and rounded once,
  round-to-nearest-even, to bfloat16 for the bf16 workloads;
* padding lengths are integers drawn uniformly from [1024, 4096] (inclusive),
  or from a caller-given range for small shapes;
* a block layout keeps each 64x64 tile independently with probability 0.25
  and always keeps the diagonal tiles.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

T_Q, T_K, T_V, T_DO, T_LEN, T_LAYOUT, T_DENSE = range(7)


@dataclass
class Workload:
    """Shape and mask recipe of one attention problem."""

    name: str
    dtype: str  # "f32", "bf16" or "fp8" (OCP e4m3 inputs, forward only)
    batch: int
    heads_q: int
    heads_kv: int
    seq_q: int
    seq_k: int
    head_dim: int
    mask: str  # "none", "causal", "padding", "block"
    backward: bool = False
    len_range: tuple = (1024, 4096)
    block: int = 64
    keep_prob: float = 0.25
    layout_per_head: bool = False
    scale: Optional[float] = None
    extra: dict = field(default_factory=dict)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)


# The five workloads the method is measured on: shapes, dtypes and masks.
WORKLOADS = {
    1: Workload("fwd_f32_b1_h2_s64_d64_none", "f32", 1, 2, 2, 64, 64, 64, "none"),
    2: Workload("fwd_bf16_b4_h16_s2048_d64_causal", "bf16", 4, 16, 16, 2048, 2048, 64, "causal"),
    3: Workload("fwd_bf16_b2_h32_s4096_d128_padding", "bf16", 2, 32, 32, 4096, 4096, 128, "padding"),
    4: Workload("fwd_bf16_b1_hq32_hkv8_s8192_d128_causal_gqa", "bf16", 1, 32, 8, 8192, 8192, 128, "causal"),
    5: Workload("fwdbwd_bf16_b2_h16_s4096_d128_block64_p025", "bf16", 2, 16, 16, 4096, 4096, 128, "block",
                backward=True),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def _normal(shape, seed: int, dtype: str) -> torch.Tensor:
    x = torch.randn(*shape, generator=_gen(seed), dtype=torch.float32)
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    elif dtype == "fp8":
        x = x.to(torch.float8_e4m3fn)   # round to nearest even; N(0, 1) stays far below 448
    return x


def make_inputs(w: Workload, seed_base: int, with_do: bool = False) -> dict:
    """Host tensors for workload ``w``; tensor t is seeded ``seed_base + t``.

    Returns a dict with q, k, v (and do), lengths (int32 [batch] or None),
    layout (uint8 [nb_q, nb_k], or [batch, heads_q, nb_q, nb_k] when
    ``w.layout_per_head``; None unless the mask is "block"), dense (uint8
    [seq_q, seq_k], or per (batch, head) likewise; only for the "dense" mask) and scale.
    """
    out = {
        "q": _normal((w.batch, w.heads_q, w.seq_q, w.head_dim), seed_base + T_Q, w.dtype),
        "k": _normal((w.batch, w.heads_kv, w.seq_k, w.head_dim), seed_base + T_K, w.dtype),
        "v": _normal((w.batch, w.heads_kv, w.seq_k, w.head_dim), seed_base + T_V, w.dtype),
        "lengths": None,
        "layout": None,
        "scale": w.softmax_scale,
    }
    if with_do or w.backward:
        out["do"] = _normal((w.batch, w.heads_q, w.seq_q, w.head_dim), seed_base + T_DO, w.dtype)
    if w.mask == "padding":
        lo, hi = w.len_range
        out["lengths"] = torch.randint(lo, hi + 1, (w.batch,), generator=_gen(seed_base + T_LEN),
                                       dtype=torch.int32)
    if w.mask == "block":
        nbq = -(-w.seq_q // w.block)
        nbk = -(-w.seq_k // w.block)
        shape = (w.batch, w.heads_q, nbq, nbk) if w.layout_per_head else (nbq, nbk)
        keep = torch.rand(*shape, generator=_gen(seed_base + T_LAYOUT)) < w.keep_prob
        diag = torch.arange(min(nbq, nbk))
        keep[..., diag, diag] = True
        out["layout"] = keep.to(torch.uint8).contiguous()
    if w.mask == "dense":
        # element mask: each pair kept with probability keep_prob, inside 64x64 blocks that are
        # themselves kept with probability 0.7 (so whole blocks are hidden too)
        shape = (w.batch, w.heads_q, w.seq_q, w.seq_k) if w.layout_per_head else (w.seq_q, w.seq_k)
        g = _gen(seed_base + T_DENSE)
        keep = torch.rand(*shape, generator=g) < w.keep_prob
        nbq = -(-w.seq_q // w.block)
        nbk = -(-w.seq_k // w.block)
        blocks = torch.rand(*shape[:-2], nbq, nbk, generator=g) < 0.7
        blocks = blocks.repeat_interleave(w.block, dim=-2).repeat_interleave(w.block, dim=-1)
        keep &= blocks[..., :w.seq_q, :w.seq_k]
        out["dense"] = keep.to(torch.uint8).contiguous()
    return out


def workload_inputs(config: int, with_do: bool = False) -> dict:
    """Inputs of one of the five measured workloads, seeded ``1000 * config + t``."""
    return make_inputs(WORKLOADS[config], 1000 * config, with_do=with_do)
