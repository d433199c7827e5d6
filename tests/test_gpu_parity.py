"""GPU parity: the HIP path against the fp64 oracle on identical seeded inputs.

Every call goes through the C ABI (``io_aware_amd`` is a ctypes binding).
Tolerances on O and LSE (absolute, after widening the GPU outputs to fp64):

* float32 path: max |O - O_ref| <= 1e-5;
* fp16 / bf16 paths: max |O - O_ref| <= 2e-2 and mean |O - O_ref| <= 2e-3;
* LSE: max |LSE - LSE_ref| <= 1e-3 on every path.

Small and medium cases are compared in full; the full-size workloads (the
same launch configuration bench.py times) are compared on a deterministic
sample of rows that includes first/last rows and tile boundaries.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import fa_inputs
import oracle

pytestmark = pytest.mark.gpu

from parity_util import DEV, LSE_TOL, TOL, compare, note, to_dev  # noqa: E402


@pytest.fixture(scope="module")
def fa():
    import io_aware_amd
    return io_aware_amd


def run_full(fa, B, H, Nq, Nk, d, dtype, causal, seed, q_sigma=1.0, label=None):
    label = label or "B%d H%d Nq%d Nk%d d%d %s causal=%d" % (B, H, Nq, Nk, d, dtype, causal)
    note("case " + label)
    q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, dtype, seed, q_sigma)
    scale = fa_inputs.default_scale(d)
    qd, kd, vd = to_dev(q, k, v)
    out, lse = fa.fa_fwd(qd, kd, vd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(q, k, v, scale, causal)
    compare(out, lse, ref_o, ref_l, dtype, label)
    return q, k, v, out, lse


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def test_single_head_f32(fa):
    w = fa_inputs.WORKLOADS["single_head_f32_n256_d64"]
    run_full(fa, w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.causal, w.seed, label=w.name)


def test_ragged_causal_f16(fa):
    w = fa_inputs.WORKLOADS["ragged_causal_f16_b2h8_n1000_d64"]
    run_full(fa, w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.causal, w.seed, label=w.name)


@pytest.mark.parametrize("name", ["prefill_causal_bf16_b8h16_n4096_d128", "long_bf16_b1h32_n16384_d128_qsigma8"])
def test_full_size_prefill_every_row(fa, name):
    """Every one of the 524288 output rows of the two full-size prefill
    workloads against the fp64 oracle (about 6 s and 47 s of oracle time on
    16 cores).  The bound is a maximum over all rows: with large score
    spread a few hundred thousand rows hold a handful near the limit, which
    a sample of rows can miss."""
    w = fa_inputs.WORKLOADS[name]
    note("case %s (all rows)" % name)
    q, k, v = fa_inputs.make_workload(w)
    qd, kd, vd = to_dev(q, k, v)
    out, lse = fa.fa_fwd(qd, kd, vd, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    del qd, kd, vd
    ref_o, ref_l = oracle.attention(q, k, v, w.scale, w.causal)
    compare(out, lse, ref_o, ref_l, w.dtype, name)


@pytest.mark.parametrize("name,nrows,seed", [("prefill_causal_bf16_b8h16_n4096_d128", 3000, None),
                                             ("long_bf16_b1h32_n16384_d128_qsigma8", 1500, None),
                                             ("long_bf16_b1h32_n16384_d128_qsigma8", 1500, 2004),
                                             ("long_bf16_b1h32_n16384_d128_qsigma8", 1500, 3004)])
def test_full_size_prefill_sampled_rows(fa, name, nrows, seed):
    """The full-size workloads on a sample of rows; the long workload (score
    spread 8x, the thinnest margin to the bound) also on two more seeds."""
    import dataclasses
    w = fa_inputs.WORKLOADS[name]
    if seed is not None:
        w = dataclasses.replace(w, seed=seed)
    note("case %s seed %d (sampled %d rows)" % (name, w.seed, nrows))
    q, k, v = fa_inputs.make_workload(w)
    qd, kd, vd = to_dev(q, k, v)
    out, lse = fa.fa_fwd(qd, kd, vd, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    rows = fa_inputs.sample_rows(w.B, w.H, w.Nq, nrows, seed=w.seed)
    ref_o, ref_l = oracle.attention(q, k, v, w.scale, w.causal, rows=rows)
    o = out.reshape(-1, w.d)[torch.from_numpy(rows).to(DEV)]
    l = lse.reshape(-1)[torch.from_numpy(rows).to(DEV)]
    compare(o, l, ref_o, ref_l, w.dtype, name)
    # every output row is finite, not only the sampled ones
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_decode_split32_full(fa):
    w = fa_inputs.WORKLOADS["decode_bf16_b16h32_nk8192_d128_split32"]
    note("case " + w.name)
    q, k, v = fa_inputs.make_workload(w)
    qd, kd, vd = to_dev(q, k, v)
    ref_o, ref_l = oracle.attention(q, k, v, w.scale, False)
    out, lse = fa.fa_fwd_splitkv(qd, kd, vd, w.num_splits, scale=w.scale)
    torch.cuda.synchronize()
    compare(out, lse, ref_o, ref_l, w.dtype, w.name + " (fa_fwd_splitkv)")
    out2, lse2 = fa.fa_fwd(qd, kd, vd, scale=w.scale)   # default splits: 32 for 8192 keys
    torch.cuda.synchronize()
    assert fa.fa_default_num_splits(w.Nk) == w.num_splits
    assert torch.equal(out2, out) and torch.equal(lse2, lse)


# ---------------------------------------------------------------------------
# Ragged shapes spanning several tiles, every head dim and type
# ---------------------------------------------------------------------------

SHAPES = [(1, 2, 300, 517), (2, 1, 517, 300), (1, 1, 129, 64), (1, 3, 64, 1), (1, 1, 1, 77),
          (1, 2, 255, 255), (1, 1, 513, 513)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("split", ["never", "auto"])
def test_ragged_shapes(fa, dtype, d, causal, split, monkeypatch):
    """Small grids: "auto" lets fa_fwd split the key range (these grids are
    below the split threshold), "never" keeps one workgroup per Q block."""
    if split == "never":
        monkeypatch.setenv("FA_PREFILL_SPLIT", "0")
        monkeypatch.setenv("FA_F32_SPLIT", "0")
    else:
        monkeypatch.delenv("FA_PREFILL_SPLIT", raising=False)
        monkeypatch.delenv("FA_F32_SPLIT", raising=False)
    for i, (B, H, Nq, Nk) in enumerate(SHAPES):
        run_full(fa, B, H, Nq, Nk, d, dtype, causal, seed=100 + i + 10 * d,
                 label="B%d H%d Nq%d Nk%d d%d %s causal=%d split=%s" % (B, H, Nq, Nk, d, dtype, causal, split))


@pytest.mark.parametrize("shape_id", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("split", ["0", "3"])
def test_every_prefill_tile_shape(fa, shape_id, split, monkeypatch):
    monkeypatch.setenv("FA_PREFILL_SHAPE", str(shape_id))
    monkeypatch.setenv("FA_PREFILL_SPLIT", split)
    for d in (64, 128):
        for causal in (False, True):
            run_full(fa, 1, 2, 700, 700, d, "bf16", causal, seed=7 + d, q_sigma=4.0,
                     label="shape %d d%d causal=%d split=%s" % (shape_id, d, causal, split))


def test_pipelined_schedule_matches_default(fa, monkeypatch):
    """FA_PREFILL_PIPE=1 (the next tile's S^T chain beside this tile's
    softmax, two waves per SIMD) does per element the arithmetic of the
    default schedule in the same order: dense, split and packed launches give
    the default's outputs bit for bit, over ragged tiles, both masks, both
    16-bit types and both head dims of 32-key tiles (shape 3, forced: small
    grids would take the key-split shapes, d = 64 the 64-key tiles)."""
    monkeypatch.setenv("FA_PREFILL_SHAPE", "3")
    dense = [(1, 2, 300, 517, 128, "bf16", True, None), (2, 1, 517, 300, 64, "f16", False, None),
             (1, 3, 64, 1, 128, "bf16", False, None), (1, 2, 700, 700, 128, "f16", True, "3"),
             (1, 1, 1500, 333, 64, "bf16", True, "2"), (1, 2, 1000, 1000, 128, "bf16", False, "5")]
    for i, (B, H, Nq, Nk, d, dtype, causal, split) in enumerate(dense):
        label = "pipe B%d H%d Nq%d Nk%d d%d %s causal=%d split=%s" % (B, H, Nq, Nk, d, dtype, causal, split)
        note("case " + label)
        q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, dtype, seed=1500 + i, q_sigma=4.0)
        qd, kd, vd = to_dev(q, k, v)
        if split is None:
            monkeypatch.setenv("FA_PREFILL_SPLIT", "0")
        else:
            monkeypatch.setenv("FA_PREFILL_SPLIT", split)
        monkeypatch.delenv("FA_PREFILL_PIPE", raising=False)
        o0, l0 = fa.fa_fwd(qd, kd, vd, causal=causal)
        monkeypatch.setenv("FA_PREFILL_PIPE", "1")
        o1, l1 = fa.fa_fwd(qd, kd, vd, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(l0, l1), label
        if i == 0:
            ref_o, ref_l = oracle.attention(q, k, v, fa_inputs.default_scale(d), causal)
            compare(o1, l1, ref_o, ref_l, dtype, label)
    w = fa_inputs.VarlenWorkload("pipe varlen", 7, 3, 128, "bf16", True, 1520, 1, 400, edge=True, same_kv=False)
    q, k, v, cq, ck = fa_inputs.make_varlen(w)
    args = to_dev(q, k, v, cq, ck)
    monkeypatch.delenv("FA_PREFILL_PIPE", raising=False)
    o0, l0 = fa.fa_fwd_varlen(*args, scale=w.scale, causal=True)
    monkeypatch.setenv("FA_PREFILL_PIPE", "1")
    o1, l1 = fa.fa_fwd_varlen(*args, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1), "pipe varlen"


@pytest.mark.parametrize("split", ["2", "5", "64"])
def test_split_prefill_chunk_counts(fa, split, monkeypatch):
    """The split path at forced chunk counts (64 is capped at one tile per
    chunk): ragged key counts, masks, key counts below and above the query
    count, large score magnitudes."""
    monkeypatch.setenv("FA_PREFILL_SPLIT", split)
    cases = [(1, 2, 1000, 1000, 64, "f16", True), (2, 1, 333, 1500, 128, "bf16", False),
             (1, 1, 1500, 333, 128, "bf16", True), (1, 3, 77, 4097, 64, "bf16", True),
             (1, 1, 640, 640, 32, "f16", False)]
    for i, (B, H, Nq, Nk, d, dtype, causal) in enumerate(cases):
        run_full(fa, B, H, Nq, Nk, d, dtype, causal, seed=700 + i, q_sigma=4.0,
                 label="split=%s B%d H%d Nq%d Nk%d d%d %s causal=%d" % (split, B, H, Nq, Nk, d, dtype, causal))


@pytest.mark.parametrize("B,H,Nq,Nk,d,dtype,causal,chunks", [
    (1, 2, 300, 5000, 64, "bf16", False, 9),     # grid 6, 79 tiles of 64 keys: 9 chunks of 9 tiles
    (1, 1, 2500, 6000, 128, "bf16", True, 10),   # grid 20; the mask leaves 2560 keys = 80 tiles of 32
    (1, 4, 500, 2100, 32, "f16", False, 1),      # grid 16, 33 tiles: under 64, the waves split the keys instead
    (2, 4, 1000, 1000, 64, "f16", True, 1),      # 16 tiles per Q block: too short to split
    (3, 48, 128, 2048, 32, "f16", False, 1),     # grid 144 with 32 tiles: chunks would share CUs
])
def test_split_prefill_automatic_choice(fa, B, H, Nq, Nk, d, dtype, causal, chunks, monkeypatch):
    """Without FA_PREFILL_SPLIT, a grid under 512 workgroups whose Q blocks
    read at least 64 K/V tiles (256 above 128 workgroups) is split into
    min(ceil(512 / grid), tiles / 8, 64) chunks (then as many as whole-tile
    chunks need): parity with the oracle, and bitwise the result of asking
    for that chunk count."""
    monkeypatch.delenv("FA_PREFILL_SPLIT", raising=False)
    q, k, v, _, _ = run_full(fa, B, H, Nq, Nk, d, dtype, causal, seed=760 + d, q_sigma=4.0,
                       label="auto split B%d H%d Nq%d Nk%d d%d %s causal=%d" % (B, H, Nq, Nk, d, dtype, causal))
    qd, kd, vd = to_dev(q, k, v)
    auto = fa.fa_fwd(qd, kd, vd, causal=causal)
    monkeypatch.setenv("FA_PREFILL_SPLIT", str(chunks))
    forced = fa.fa_fwd(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(auto[0], forced[0]) and torch.equal(auto[1], forced[1])


@pytest.mark.parametrize("split", ["0", "2", "3", "7", "64"])
def test_f32_split_chunk_counts(fa, split, monkeypatch):
    """The float32 path with its key range cut into at most n chunks of
    whole 32-key blocks (0: never split; 64 is capped at one block per
    chunk), then combined: ragged key counts, both masks, keys below and
    above the query count (chunks past a causal row block's keys are
    empty), every head dim; max |dO| <= 1e-5 as for the unsplit path."""
    monkeypatch.setenv("FA_F32_SPLIT", split)
    cases = [(1, 1, 256, 256, 64, False), (1, 2, 300, 517, 32, True), (2, 1, 517, 300, 128, True),
             (1, 1, 129, 1000, 64, True), (1, 3, 70, 700, 128, False), (1, 1, 1, 200, 64, False)]
    for i, (B, H, Nq, Nk, d, causal) in enumerate(cases):
        run_full(fa, B, H, Nq, Nk, d, "f32", causal, seed=820 + i,
                 label="f32 split=%s B%d H%d Nq%d Nk%d d%d causal=%d" % (split, B, H, Nq, Nk, d, causal))


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,chunks", [
    (1, 1, 256, 256, 64, False, 8),     # the single-head workload: grid 4, 8 blocks: one block per chunk
    (1, 2, 300, 5000, 32, False, 40),   # grid 10: 52 chunks wanted, 157 blocks: 40 chunks of 4 blocks
    (4, 64, 64, 512, 64, True, 1),      # grid 256: no split
])
def test_f32_split_automatic_choice(fa, B, H, Nq, Nk, d, causal, chunks, monkeypatch):
    """Without FA_F32_SPLIT a float32 grid below 256 workgroups is split
    into min(ceil(512 / grid), 64) chunks of whole 32-key blocks (then as
    many as whole-block chunks need): parity with the oracle, and bitwise
    the result of asking for that chunk count."""
    monkeypatch.delenv("FA_F32_SPLIT", raising=False)
    q, k, v, _, _ = run_full(fa, B, H, Nq, Nk, d, "f32", causal, seed=840 + d,
                             label="f32 auto split B%d H%d Nq%d Nk%d d%d causal=%d" % (B, H, Nq, Nk, d, causal))
    qd, kd, vd = to_dev(q, k, v)
    auto = fa.fa_fwd(qd, kd, vd, causal=causal)
    monkeypatch.setenv("FA_F32_SPLIT", str(chunks))
    forced = fa.fa_fwd(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(auto[0], forced[0]) and torch.equal(auto[1], forced[1])


@pytest.mark.parametrize("B,H,Nq,Nk,d,dtype,causal,shape", [
    (2, 8, 1000, 1000, 64, "f16", True, 5),       # the ragged workload: grid 128, 16 tiles: four-way key split
    (1, 4, 700, 900, 32, "bf16", False, 5),       # d = 32: four-way with 64-key tiles
    (2, 8, 1000, 1000, 128, "bf16", True, 4),     # d = 128: two-way
    (1, 40, 600, 1500, 64, "bf16", False, 4),     # grid 200, between 128 and 256: two-way
    (4, 16, 1000, 1000, 64, "f16", True, None),   # grid 512: no key split
    (2, 8, 300, 300, 64, "f16", True, None),      # 5 tiles per Q block: no key split
])
def test_key_split_automatic_choice(fa, B, H, Nq, Nk, d, dtype, causal, shape, monkeypatch):
    """A dense grid below one workgroup per CU whose longest Q block reads
    at least 8 K/V tiles splits each query group's key loop over 2 or 4
    waves of the workgroup (merged through LDS): parity with the oracle, and
    bitwise the result of forcing that shape (or the default one)."""
    monkeypatch.delenv("FA_PREFILL_SPLIT", raising=False)
    monkeypatch.delenv("FA_PREFILL_SHAPE", raising=False)
    q, k, v, _, _ = run_full(fa, B, H, Nq, Nk, d, dtype, causal, seed=780 + d, q_sigma=3.0,
                             label="auto key split B%d H%d Nq%d Nk%d d%d %s causal=%d" % (B, H, Nq, Nk, d, dtype, causal))
    qd, kd, vd = to_dev(q, k, v)
    auto = fa.fa_fwd(qd, kd, vd, causal=causal)
    monkeypatch.setenv("FA_PREFILL_SHAPE", str(shape if shape is not None else (3 if d == 128 else 0)))
    forced = fa.fa_fwd(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(auto[0], forced[0]) and torch.equal(auto[1], forced[1])


@pytest.mark.parametrize("shape_id", [0, 3, 4, 5])
def test_prefill_shape_edge_cases(fa, shape_id, monkeypatch):
    """Key counts below, at and above the query count, single keys and
    queries, partial blocks of queries and keys, at d = 128 for the 64-key
    tile shape and the default 32-key tile shape."""
    monkeypatch.setenv("FA_PREFILL_SHAPE", str(shape_id))
    cases = [(1, 2, 300, 1000), (1, 2, 1000, 300), (2, 1, 257, 31), (1, 1, 64, 1), (1, 1, 1, 33),
             (1, 1, 512, 512), (1, 1, 33, 2000)]
    for i, (B, H, Nq, Nk) in enumerate(cases):
        for causal in (False, True):
            run_full(fa, B, H, Nq, Nk, 128, "bf16", causal, seed=900 + i, q_sigma=2.0,
                     label="shape %d B%d H%d Nq%d Nk%d causal=%d" % (shape_id, B, H, Nq, Nk, causal))


def test_triton_page_regression(fa):
    """The fp16 shapes and seed of the Triton page's test; its bound is
    max-abs < 1e-3 against an fp16 torch reference, here against fp64."""
    import json
    spec = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "triton_page_test.json")))
    for (Nq, Nk, d) in spec["shapes_nq_nk_d"]:
        q, k, v = fa_inputs.make_qkv(1, 1, Nq, Nk, d, "f16", spec["seed"])
        scale = fa_inputs.default_scale(d)
        out, lse = fa.fa_fwd(*to_dev(q, k, v), scale=scale)
        torch.cuda.synchronize()
        ref_o, _ = oracle.attention(q, k, v, scale, False)
        err = np.abs(out.float().cpu().numpy() - ref_o).max()
        note("triton page case %dx%dx%d: max|dO| = %.3e" % (Nq, Nk, d, err))
        assert err < spec["max_abs_tol"]


# ---------------------------------------------------------------------------
# Split-KV edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("Nk,S", [(8192, 1), (1000, 7), (50, 64), (1, 1), (513, 32), (4096, 1024)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_splitkv_edge_cases(fa, Nk, S, dtype):
    note("case splitkv Nk=%d S=%d %s" % (Nk, S, dtype))
    q, k, v = fa_inputs.make_qkv(2, 3, 1, Nk, 128, dtype, seed=Nk + S, q_sigma=3.0)
    scale = fa_inputs.default_scale(128)
    out, lse = fa.fa_fwd_splitkv(*to_dev(q, k, v), S, scale=scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(q, k, v, scale, False)
    compare(out, lse, ref_o, ref_l, dtype, "splitkv Nk=%d S=%d" % (Nk, S))


# ---------------------------------------------------------------------------
# Invariants, determinism, guard bands
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_constant_values_give_that_constant(fa, dtype):
    q, k, v = fa_inputs.make_qkv(1, 2, 333, 333, 128, dtype, seed=21, q_sigma=8.0)
    v[:] = v[:, :, :1, :]                       # every value row equal
    for causal in (False, True):
        out, _ = fa.fa_fwd(*to_dev(q, k, v), causal=causal)
        torch.cuda.synchronize()
        c = v[:, :, :1, :].float().expand_as(out).cpu()
        rel = ((out.float().cpu() - c).abs() / c.abs().clamp_min(1e-3)).max().item()
        assert rel <= 2.0 ** -7, rel        # within one unit in the last place of the 16-bit type


def test_causal_first_row_and_single_query(fa):
    q, k, v = fa_inputs.make_qkv(2, 2, 200, 200, 64, "bf16", seed=22, q_sigma=8.0)
    out, lse = fa.fa_fwd(*to_dev(q, k, v), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, 0].cpu(), v[:, :, 0])       # only key 0 is visible: P = 1 exactly
    q1 = q[:, :, :1].contiguous()
    out1, _ = fa.fa_fwd(*to_dev(q1, k, v), causal=True)      # Nq = 1 under the mask: key 0 only
    torch.cuda.synchronize()
    assert torch.equal(out1[:, :, 0].cpu(), v[:, :, 0])


def test_key_value_permutation_equivariance(fa):
    q, k, v = fa_inputs.make_qkv(1, 2, 256, 300, 128, "bf16", seed=23)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(300))
    o1, l1 = fa.fa_fwd(*to_dev(q, k, v))
    o2, l2 = fa.fa_fwd(*to_dev(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous()))
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
    assert (l1 - l2).abs().max().item() <= 1e-3


def test_bitwise_deterministic(fa):
    q, k, v = fa_inputs.make_qkv(2, 4, 1000, 1000, 128, "bf16", seed=24)
    qd, kd, vd = to_dev(q, k, v)
    for causal in (False, True):
        a = fa.fa_fwd(qd, kd, vd, causal=causal)
        b = fa.fa_fwd(qd, kd, vd, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype,Nq,Nk,causal", [("bf16", 1000, 1000, True), ("f32", 100, 70, False),
                                                ("bf16", 1, 8192, False), ("f16", 77, 33, True)])
def test_guard_bands_untouched(fa, dtype, Nq, Nk, causal):
    B, H, d = 2, 3, 128
    q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, dtype, seed=25)
    qd, kd, vd = to_dev(q, k, v)
    n_out, n_lse, pad = B * H * Nq * d, B * H * Nq, 4096
    tdt = fa_inputs.DTYPES[dtype]
    obuf = torch.full((n_out + 2 * pad,), 7.0, dtype=tdt, device=DEV)
    lbuf = torch.full((n_lse + 2 * pad,), 7.0, dtype=torch.float32, device=DEV)
    out = obuf[pad:pad + n_out].view(B, H, Nq, d)
    lse = lbuf[pad:pad + n_lse].view(B, H, Nq)
    fa.fa_fwd(qd, kd, vd, causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    for buf, n in ((obuf, n_out), (lbuf, n_lse)):
        assert (buf[:pad].float() == 7.0).all() and (buf[pad + n:].float() == 7.0).all()
    ref_o, ref_l = oracle.attention(q, k, v, fa_inputs.default_scale(d), causal)
    compare(out, lse, ref_o, ref_l, dtype, "guard bands %s" % dtype)


def _timed_on(stream, fn):
    """Events on ``stream`` around ``fn()``: elapsed ms after the stream drains."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    r = fn()
    e.record(stream)
    stream.synchronize()
    return r, s.elapsed_time(e)


@pytest.mark.parametrize("Nq", [4096, 1])
def test_side_stream(fa, Nq):
    """The entry point enqueues on the caller's stream: the current stream
    inside ``torch.cuda.stream(s)`` and the ``stream`` argument both give the
    default stream's result bit for bit, and events recorded on the side
    stream around the call span the kernels (a launch on another stream
    would leave them less than a kernel's length apart).  Nq = 1 is the
    decode path, with its per-stream library workspace."""
    B, H, Nk, d = 2, 16, 4096, 128
    q, k, v = fa_inputs.make_qkv_device(B, H, Nq, Nk, d, "bf16", seed=32, device=DEV)
    causal = Nq > 1
    main = torch.cuda.current_stream()
    for _ in range(3):                                   # warm the clocks
        fa.fa_fwd(q, k, v, causal=causal)
    # the fastest of five: host work between the event records can only add
    # to a single measurement (for the 25 us decode kernels, several-fold)
    runs = [_timed_on(main, lambda: fa.fa_fwd(q, k, v, causal=causal)) for _ in range(5)]
    (ref_o, ref_l), t_main = runs[0][0], min(t for _, t in runs)
    side = torch.cuda.Stream()                           # default priority
    side.wait_stream(main)
    with torch.cuda.stream(side):
        (o1, l1), t1 = _timed_on(side, lambda: fa.fa_fwd(q, k, v, causal=causal))
    (o2, l2), t2 = _timed_on(side, lambda: fa.fa_fwd(q, k, v, causal=causal, stream=side))
    torch.cuda.synchronize()
    for o, l in ((o1, l1), (o2, l2)):
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    assert t1 >= 0.5 * t_main and t2 >= 0.5 * t_main, (t_main, t1, t2)


def test_release_workspace_after_growth(fa):
    """Grow the library workspace of two streams (the replaced buffers are
    retired, not freed), release everything, and decode again: the release
    returns FA_OK twice in a row and later calls allocate afresh and give
    the same results bit for bit."""
    side = torch.cuda.Stream()
    shapes = [(2, 4, 1024), (4, 8, 30000), (8, 16, 8192)]   # split workspaces of 16 KB, 1 MB, 2.1 MB
    results = {}
    for B, H, Nk in shapes:
        q, k, v = fa_inputs.make_qkv_device(B, H, 1, Nk, 128, "bf16", seed=Nk, device=DEV)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            o_side, l_side = fa.fa_fwd(q, k, v)
        o, l = fa.fa_fwd(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o, o_side) and torch.equal(l, l_side)
        results[(B, H, Nk)] = (q, k, v, o, l)
    fa.fa_release_workspace()   # raises FAError unless FA_OK
    fa.fa_release_workspace()
    for (B, H, Nk), (q, k, v, o, l) in results.items():
        o2, l2 = fa.fa_fwd(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(l, l2)


def test_lse_optional(fa):
    q, k, v = fa_inputs.make_qkv(1, 2, 100, 100, 64, "bf16", seed=26)
    qd, kd, vd = to_dev(q, k, v)
    o1, _ = fa.fa_fwd(qd, kd, vd, return_lse=False)
    o2, _ = fa.fa_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_binding_rejects_mismatched_outputs(fa):
    """An output of the wrong size, type or layout is refused before any
    launch (the library cannot see buffer sizes), and the refused tensors are
    left as they were."""
    q, k, v = fa_inputs.make_qkv(1, 2, 100, 80, 64, "bf16", seed=27)
    qd, kd, vd = to_dev(q, k, v)
    out, lse = fa.fa_fwd(qd, kd, vd)
    g = torch.randn_like(qd)
    small = torch.full((1, 2, 99, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    cases = [
        lambda: fa.fa_fwd(qd, kd, vd, out=small),
        lambda: fa.fa_fwd(qd, kd, vd, out=torch.empty_like(qd, dtype=torch.float16)),
        lambda: fa.fa_fwd(qd, kd, vd, lse=torch.empty((1, 2, 100), dtype=torch.float16, device=DEV)),
        lambda: fa.fa_fwd_noalloc(qd, kd, vd, torch.empty((1, 100, 2, 64), dtype=torch.bfloat16,
                                                          device=DEV).transpose(1, 2)),
        lambda: fa.fa_bwd(qd, kd, vd, out, g, lse, dk=torch.empty_like(qd)),
        lambda: fa.fa_bwd(qd, kd, vd, out, g, lse, workspace=torch.empty(1 << 20, dtype=torch.uint8)),
    ]
    for call in cases:
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()
    assert (small.float() == 3.0).all()


def test_large_values_and_rising_scores_stay_finite(fa):
    """bf16 values near 2^94 with scores that climb slowly along 16384 keys:
    the lazy rescale bounds the running sum of P (not each tile's), so the
    float32 accumulator stays finite; O is compared after division by 2^94
    (exact: both sides scale by a power of two)."""
    note("case rising scores, values near 2^94")
    q, k, v = fa_inputs.make_rising_scores(16384, 128)
    scale = fa_inputs.default_scale(128)
    out, lse = fa.fa_fwd(*to_dev(q, k, v), scale=scale, causal=False)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(q, k, v, scale, False)
    o = out.float().cpu().numpy().astype(np.float64) / 2.0 ** 94
    assert np.isfinite(o).all()
    # every output is near 1.05, where rounding to bf16 alone leaves a mean
    # error of about 2^-9: the max and LSE bars apply, not the mean bar of
    # outputs of unit spread
    err = np.abs(o - ref_o / 2.0 ** 94)
    lerr = np.abs(lse.cpu().numpy() - ref_l)
    note("rising scores, values / 2^94: max|dO|=%.3e max|dLSE|=%.3e" % (err.max(), lerr.max()))
    assert err.max() <= TOL["bf16"][0] and lerr.max() <= LSE_TOL
