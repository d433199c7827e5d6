"""Seeded synthetic inputs for the FlashAttention forward workloads.

Both the HIP path (through ``io_aware_amd``) and the fp64 oracle consume the
tensors made here; this module holds no attention arithmetic.  Recipe, the
same for every workload:

* a CPU ``torch.Generator`` seeded with the workload's seed;
* ``torch.randn`` in float32, drawn in the order q, k, v, each with its full
  [B, H, N, d] shape;
* q multiplied by ``q_sigma`` (1 unless stated: the long non-causal workload
  uses 8 so that scores are large and the running max moves a lot);
* a cast to the workload dtype with round-to-nearest-even (torch's ``.to``).

The same rounded tensors go to the GPU and, widened exactly to float32, to
the oracle.  The softmax scale is 1/sqrt(d) rounded to float32, and that
float32 value is what both sides receive.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    seed: int
    q_sigma: float = 1.0
    num_splits: int = 0          # > 0: run through the explicit split-KV entry point
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]


def default_scale(d: int) -> float:
    """1/sqrt(d), rounded to float32 (the value the C entry point receives)."""
    return float(np.float32(1.0 / math.sqrt(d)))


# The workloads: single-head fp32; ragged causal fp16; causal bf16 prefill;
# long non-causal bf16 with large scores; single-token bf16 decode split 32 ways.
WORKLOADS = {
    w.name: w for w in [
        Workload("single_head_f32_n256_d64", 1, 1, 256, 256, 64, "f32", False, 1001,
                 note="Br = Bc = 64"),
        Workload("ragged_causal_f16_b2h8_n1000_d64", 2, 8, 1000, 1000, 64, "f16", True, 1002),
        Workload("prefill_causal_bf16_b8h16_n4096_d128", 8, 16, 4096, 4096, 128, "bf16", True, 1003),
        Workload("long_bf16_b1h32_n16384_d128_qsigma8", 1, 32, 16384, 16384, 128, "bf16", False, 1004,
                 q_sigma=8.0),
        Workload("decode_bf16_b16h32_nk8192_d128_split32", 16, 32, 1, 8192, 128, "bf16", False, 1005,
                 num_splits=32),
    ]
}

# The fp16 shapes of the Triton page's own test (seed 42, 2-D per-head inputs,
# seqlen_q x seqlen_k x head_dim), run here as B = H = 1.
TRITON_PAGE_SHAPES = [(256, 256, 64), (128, 256, 64), (64, 64, 32)]


def make_qkv(B: int, H: int, Nq: int, Nk: int, d: int, dtype, seed: int,
             q_sigma: float = 1.0):
    """q [B,H,Nq,d], k and v [B,H,Nk,d] on the CPU, in ``dtype``."""
    if isinstance(dtype, str):
        dtype = DTYPES[dtype]
    g = torch.Generator().manual_seed(int(seed))
    q = torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32)
    if q_sigma != 1.0:
        q.mul_(q_sigma)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def make_workload(w: Workload):
    return make_qkv(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed, w.q_sigma)


def sample_rows(B: int, H: int, Nq: int, count: int, seed: int, tile: int = 64):
    """A deterministic sample of flat query rows (b*H + h)*Nq + i.

    It always holds, for a spread of (b, h) pairs, the first and last rows
    and the rows on both sides of tile boundaries (where masks and ragged
    tails change), then fills up to ``count`` with uniformly drawn rows.
    """
    rng = np.random.default_rng(seed)
    BH = B * H
    picked = set()
    heads = sorted(set([0, BH - 1] + list(rng.integers(0, BH, size=min(BH, 8)))))
    special = {0, 1, Nq - 1, Nq - 2}
    for t in range(tile, Nq, tile * max(1, Nq // (tile * 8))):
        special.update({t - 1, t})
    special = {i for i in special if 0 <= i < Nq}
    for bh in heads:
        for i in special:
            picked.add(bh * Nq + i)
    total = BH * Nq
    while len(picked) < min(count, total):
        picked.add(int(rng.integers(0, total)))
    return np.array(sorted(picked), dtype=np.int64)
