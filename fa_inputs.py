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
    backward: bool = False       # the workload of the backward pass (forward output and LSE, then gradients)
    fp8: bool = False            # the FP8 forward on the quantised pack (incoherent processing on)
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
        Workload("bwd_causal_bf16_b8h16_n4096_d128", 8, 16, 4096, 4096, 128, "bf16", True, 1008, backward=True,
                 note="the causal prefill shapes, backward"),
        Workload("fp8_causal_b8h16_n4096_d128", 8, 16, 4096, 4096, 128, "bf16", True, 1011, fp8=True,
                 note="the causal prefill shapes, E4M3 inputs"),
    ]
}



@dataclass(frozen=True)
class PagedWorkload:
    """Single-token decode over a paged K/V cache [num_blocks, H, block_size, d]."""
    name: str
    B: int
    H: int
    d: int
    block_size: int
    max_len: int                 # keys of the longest sequence; the table has ceil(max_len/block_size) columns
    dtype: str
    seed: int
    num_splits: int
    lens: str = "full"           # "full": every sequence max_len keys; "mixed": drawn lengths, edge cases included
    hole_frac: float = 0.0       # fraction of a sequence's logical blocks left unallocated (table entry -1)
    spare_blocks: int = 0        # physical blocks no table entry names
    poison: bool = False         # fill every cache row no sequence reads with NaN
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]


PAGED_WORKLOADS = {
    w.name: w for w in [
        PagedWorkload(
            "paged_decode_bf16_b16h32_len8192_d128_bs16_split32", 16, 32, 128, 16, 8192, "bf16", 1006, 32,
            note="the decode workload's sizes with the cache in 16-key pages in shuffled order"),
        PagedWorkload("paged_mixed_f16_b6h4_len1000_d64_bs16_split8", 6, 4, 64, 16, 1000, "f16", 1007, 8,
                      lens="mixed", hole_frac=0.1, spare_blocks=5, poison=True),
    ]
}


def _paged_lengths(w: PagedWorkload, g):
    if w.lens == "full":
        return [w.max_len] * w.B
    bs = w.block_size
    edge = [0, 1, bs - 1, bs + 1, w.max_len]
    rest = torch.randint(1, w.max_len + 1, (w.B,), generator=g).tolist()
    return [min(w.max_len, x) for x in (edge + rest)[:w.B]]


def paged_lengths(w: PagedWorkload):
    """The sequence lengths make_paged draws (the first draws of its
    generator), without the caches."""
    return _paged_lengths(w, torch.Generator().manual_seed(int(w.seed)))


def make_paged(w: PagedWorkload):
    """(q, k_cache, v_cache, block_table, seq_lens) on the CPU.

    Recipe: a CPU generator seeded with ``w.seed`` draws, in order,
    * the sequence lengths: all ``max_len`` ("full"), or ("mixed") the edge
      lengths 0, 1, block_size - 1, block_size + 1 and max_len first, the rest
      uniform in [1, max_len];
    * a permutation of the physical blocks; each sequence takes its
      ceil(len / block_size) logical blocks from it in order, so consecutive
      logical blocks sit at unrelated physical places; unused table columns
      are -1;
    * with ``hole_frac`` > 0, that fraction of allocated table entries set to
      -1 (unallocated: their keys are skipped);
    * q [B, H, 1, d], then k_cache and v_cache [num_blocks, H, block_size, d],
      standard normal in float32, rounded to the dtype (nearest-even).
    With ``poison``, every cache row no sequence reads (spare blocks, rows of
    a last block past the sequence end, blocks of holes) is set to NaN, so a
    stray read shows up in the output.
    """
    g = torch.Generator().manual_seed(int(w.seed))
    bs = w.block_size
    max_blocks = -(-w.max_len // bs)
    lens = _paged_lengths(w, g)
    need = [-(-n // bs) for n in lens]
    num_blocks = sum(need) + w.spare_blocks
    perm = torch.randperm(max(num_blocks, 1), generator=g).tolist()
    table = torch.full((w.B, max_blocks), -1, dtype=torch.int32)
    pos = 0
    for b in range(w.B):
        for j in range(need[b]):
            table[b, j] = perm[pos]
            pos += 1
    if w.hole_frac > 0:
        drop = torch.rand((w.B, max_blocks), generator=g) < w.hole_frac
        table[drop] = -1
    q = torch.randn((w.B, w.H, 1, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((max(num_blocks, 1), w.H, bs, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((max(num_blocks, 1), w.H, bs, w.d), generator=g, dtype=torch.float32)
    if w.poison:
        used = torch.zeros((k.shape[0], bs), dtype=torch.bool)
        for b in range(w.B):
            for j in range(need[b]):
                blk = int(table[b, j])
                if blk >= 0:
                    used[blk, :min(bs, lens[b] - j * bs)] = True
        unread = ~used[:, None, :, None]
        k.masked_fill_(unread, float("nan"))
        v.masked_fill_(unread, float("nan"))
    seq_lens = torch.tensor(lens, dtype=torch.int32)
    return q.to(w.torch_dtype), k.to(w.torch_dtype), v.to(w.torch_dtype), table, seq_lens


@dataclass(frozen=True)
class VarlenWorkload:
    """A batch of packed sequences of different lengths: q [total_q, H, d],
    k and v [total_k, H, d], cumulative offsets [S + 1]."""
    name: str
    S: int
    H: int
    d: int
    dtype: str
    causal: bool
    seed: int
    min_len: int
    max_len: int
    edge: bool = False           # put the edge lengths first (see make_varlen)
    same_kv: bool = True         # key lengths equal query lengths (self-attention)
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]


VARLEN_WORKLOADS = {
    w.name: w for w in [
        VarlenWorkload("varlen_causal_bf16_s16h16_len256to8192_d128", 16, 16, 128, "bf16", True, 1009, 256, 8192,
                       note="lengths uniform in [256, 8192]: a mixed prefill batch"),
        VarlenWorkload("varlen_mixed_f16_s9h4_len0to700_d64", 9, 4, 64, "f16", True, 1010, 0, 700, edge=True,
                       same_kv=False),
    ]
}


def _varlen_lengths(w: VarlenWorkload, g):
    def lengths():
        x = torch.randint(w.min_len, w.max_len + 1, (w.S,), generator=g).tolist()
        if w.edge:
            x = ([0, 1, 127, 128, 129, w.max_len] + x)[:w.S]
        return x
    lq = lengths()
    return lq, (lq if w.same_kv else lengths())


def varlen_lengths(w: VarlenWorkload):
    """(query lengths, key lengths) as make_varlen draws them (the first
    draws of its generator), without the tensors."""
    return _varlen_lengths(w, torch.Generator().manual_seed(int(w.seed)))


def make_varlen(w: VarlenWorkload):
    """(q, k, v, cu_seqlens_q, cu_seqlens_k) on the CPU.

    Recipe: a CPU generator seeded with ``w.seed`` draws the query lengths
    (uniform in [min_len, max_len]; with ``edge`` the lengths 0, 1, 127, 128,
    129 and max_len come first), then, unless ``same_kv``, the key lengths
    the same way, then q [total_q, H, d], k and v [total_k, H, d], standard
    normal in float32, rounded to the dtype (nearest-even).  Offsets are
    int32 cumulative sums starting at 0.
    """
    g = torch.Generator().manual_seed(int(w.seed))
    lq, lk = _varlen_lengths(w, g)
    cq = torch.tensor([0] + lq, dtype=torch.int64).cumsum(0).to(torch.int32)
    ck = torch.tensor([0] + lk, dtype=torch.int64).cumsum(0).to(torch.int32)
    q = torch.randn((int(cq[-1]), w.H, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((int(ck[-1]), w.H, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((int(ck[-1]), w.H, w.d), generator=g, dtype=torch.float32)
    return q.to(w.torch_dtype), k.to(w.torch_dtype), v.to(w.torch_dtype), cq, ck


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


def make_qkv_device(B: int, H: int, Nq: int, Nk: int, d: int, dtype, seed: int, device):
    """Like make_qkv, but drawn on ``device`` by its own seeded generator
    (for tensors too large to draw on the host): q [B,H,Nq,d], k and v
    [B,H,Nk,d] standard normal in float32, rounded to ``dtype``, one head
    at a time so the float32 draw never exceeds one head."""
    if isinstance(dtype, str):
        dtype = DTYPES[dtype]
    g = torch.Generator(device=device).manual_seed(int(seed))
    out = []
    for n in (Nq, Nk, Nk):
        t = torch.empty((B, H, n, d), dtype=dtype, device=device)
        flat = t.view(B * H, n, d)
        for i in range(B * H):
            flat[i].copy_(torch.randn((n, d), generator=g, dtype=torch.float32, device=device))
        out.append(t)
    return tuple(out)


def make_workload(w: Workload):
    return make_qkv(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed, w.q_sigma)


def make_signs(d: int, seed: int):
    """The random signs of the incoherent transform: float32 [d] of +-1 from a
    CPU generator seeded with seed + 600000 (a fair coin per element)."""
    g = torch.Generator().manual_seed(int(seed) + 600000)
    return torch.where(torch.rand(d, generator=g) < 0.5, -1.0, 1.0).to(torch.float32)


def make_dout(B: int, H: int, Nq: int, d: int, dtype, seed: int):
    """The upstream gradient dO [B, H, Nq, d]: standard normal in float32 from
    its own CPU generator (seed + 500000, so it never repeats q's draws),
    rounded to ``dtype`` (nearest-even)."""
    if isinstance(dtype, str):
        dtype = DTYPES[dtype]
    g = torch.Generator().manual_seed(int(seed) + 500000)
    return torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32).to(dtype)


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


def make_rising_scores(N: int, d: int, seed: int = 77, value_exp: int = 94):
    """q [1, 1, 64, d], k and v [1, 1, N, d] in bf16 that stress the lazy
    rescale's range: every query is [1, 0, ...]; key j's first dim is
    j * 29 / (c (N - 1)) with c = scale * log2(e) at scale 1/sqrt(d) (so the
    scaled scores climb by 29 in base 2 over the sequence), its other dims
    N(0, 0.01^2); values uniform in [1, 1.1) * 2^value_exp.  Drawn from a CPU
    generator seeded with ``seed`` (k's noise, then v)."""
    g = torch.Generator().manual_seed(int(seed))
    c = float(np.float32(default_scale(d) * 1.4426950408889634))
    q = torch.zeros(64, d)
    q[:, 0] = 1.0
    k = torch.randn(N, d, generator=g) * 0.01
    k[:, 0] = torch.arange(N) * (29.0 / (c * (N - 1)))
    v = (1.0 + 0.1 * torch.rand(N, d, generator=g)) * 2.0 ** value_exp
    return tuple(t.to(torch.bfloat16)[None, None] for t in (q, k, v))
