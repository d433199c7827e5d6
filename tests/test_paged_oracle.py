"""Pins of the paged-cache oracle (``oracle.paged_decode``) on the CPU.

The paged oracle gathers the keys a block table maps and hands them to the
three-pass ``oracle.attention``, which other tests pin.  What is new here is
the gather, and these tests fix it from outside itself:

* an identity table over a cache cut from contiguous K/V gives exactly the
  contiguous result (a wrong head, row or block index breaks it);
* permuting the physical blocks, with the table rewritten to match, changes
  nothing, bit for bit;
* an unallocated entry (-1, or an index past the cache) equals deleting that
  block's keys from the contiguous K/V ("6. FlashAttention 分块逻辑",
  section 12.2 skips such blocks);
* a length that ends inside a block takes only that block's first rows;
* the page's own block-by-block online loop (``paged_attention_blocked``)
  agrees with the gather + three-pass oracle to rounding;
* no key at all gives O = 0 and LSE = -inf;
* a planted mistake (the last block taken whole) is caught.
"""
import math

import numpy as np
import pytest

import fa_inputs
import oracle
from oracle import algorithms as alg


def contiguous_case(B=3, H=2, n=70, d=16, bs=8, seed=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, 1, d)).astype(np.float32)
    k = rng.standard_normal((B, H, n, d)).astype(np.float32)
    v = rng.standard_normal((B, H, n, d)).astype(np.float32)
    return q, k, v


def to_paged(k, bs, order=None):
    """Cut [B, H, n, d] into a cache [B*nb, H, bs, d] (zero padded) with
    sequence b's block j at physical index order[b*nb + j]."""
    B, H, n, d = k.shape
    nb = -(-n // bs)
    pad = np.zeros((B, H, nb * bs, d), dtype=k.dtype)
    pad[:, :, :n] = k
    blocks = pad.reshape(B, H, nb, bs, d).transpose(0, 2, 1, 3, 4).reshape(B * nb, H, bs, d)
    if order is None:
        order = np.arange(B * nb)
    cache = np.empty_like(blocks)
    cache[order] = blocks
    table = np.asarray(order, dtype=np.int64).reshape(B, nb)
    return cache, table


def test_identity_table_equals_contiguous():
    q, k, v = contiguous_case()
    scale = 0.25
    kc, table = to_paged(k, 8)
    vc, _ = to_paged(v, 8)
    lens = np.full(3, k.shape[2])
    out, lse = oracle.paged_decode(q, kc, vc, table, lens, scale)
    ref_o, ref_l = oracle.attention(q, k, v, scale, False)
    np.testing.assert_array_equal(out, ref_o[:, :, 0])
    np.testing.assert_array_equal(lse, ref_l[:, :, 0])


def test_block_permutation_invariance():
    q, k, v = contiguous_case(seed=6)
    kc0, t0 = to_paged(k, 8)
    vc0, _ = to_paged(v, 8)
    order = np.random.default_rng(1).permutation(kc0.shape[0])
    kc1, t1 = to_paged(k, 8, order)
    vc1, _ = to_paged(v, 8, order)
    assert not np.array_equal(kc0, kc1)
    lens = np.array([70, 33, 8])
    a = oracle.paged_decode(q, kc0, vc0, t0, lens, 0.3)
    b = oracle.paged_decode(q, kc1, vc1, t1, lens, 0.3)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("bad", [-1, -7, 9999])
def test_unallocated_block_equals_deleted_keys(bad):
    q, k, v = contiguous_case(seed=7)
    bs = 8
    kc, table = to_paged(k, bs)
    vc, _ = to_paged(v, bs)
    table = table.copy()
    table[1, 2] = bad               # keys 16..23 of sequence 1
    table[2, 0] = bad               # keys 0..7 of sequence 2
    lens = np.full(3, 70)
    out, lse = oracle.paged_decode(q, kc, vc, table, lens, 0.2)
    keep = {0: np.arange(70), 1: np.r_[0:16, 24:70], 2: np.arange(8, 70)}
    for b in range(3):
        ro, rl = oracle.attention(q[b:b + 1], k[b:b + 1, :, keep[b]], v[b:b + 1, :, keep[b]], 0.2, False)
        np.testing.assert_array_equal(out[b], ro[0, :, 0])
        np.testing.assert_array_equal(lse[b], rl[0, :, 0])


@pytest.mark.parametrize("n", [1, 7, 8, 9, 69, 70])
def test_length_inside_a_block_takes_first_rows(n):
    q, k, v = contiguous_case(seed=8)
    kc, table = to_paged(k, 8)
    vc, _ = to_paged(v, 8)
    # rows past n (inside the last block, and later blocks) hold NaN: never read
    kc = kc.copy()
    vc = vc.copy()
    nb = table.shape[1]
    for b in range(3):
        for j in range(nb):
            lo = max(0, n - j * 8)
            kc[table[b, j], :, lo:] = np.nan
            vc[table[b, j], :, lo:] = np.nan
    out, lse = oracle.paged_decode(q, kc, vc, table, np.full(3, n), 0.2)
    ro, rl = oracle.attention(q, k[:, :, :n], v[:, :, :n], 0.2, False)
    np.testing.assert_array_equal(out, ro[:, :, 0])
    np.testing.assert_array_equal(lse, rl[:, :, 0])


def test_length_is_clamped_to_the_table():
    q, k, v = contiguous_case(seed=9, n=64)
    kc, table = to_paged(k, 8)
    vc, _ = to_paged(v, 8)
    big = oracle.paged_decode(q, kc, vc, table, np.full(3, 10 ** 6), 0.2)
    full = oracle.paged_decode(q, kc, vc, table, np.full(3, 64), 0.2)
    np.testing.assert_array_equal(big[0], full[0])
    neg = oracle.paged_decode(q, kc, vc, table, np.full(3, -5), 0.2)
    assert (neg[0] == 0).all() and np.isneginf(neg[1]).all()


def test_no_key_gives_zero_and_minus_inf():
    q, k, v = contiguous_case(seed=10)
    kc, table = to_paged(k, 8)
    vc, _ = to_paged(v, 8)
    t = table.copy()
    t[1, :] = -1
    out, lse = oracle.paged_decode(q, kc, vc, t, np.array([0, 70, 70]), 0.2)
    assert (out[:2] == 0).all() and np.isneginf(lse[:2]).all()
    assert np.isfinite(lse[2]).all()
    o, l = alg.paged_attention_blocked(q[0, 0, 0], kc[:, 0], vc[:, 0], t[1], 70, 0.2)
    assert (o == 0).all() and l == -math.inf


def test_page_loop_agrees_with_gather_oracle():
    w = fa_inputs.PagedWorkload("t", 6, 3, 32, 16, 300, "f32", 77, 4, lens="mixed", hole_frac=0.2,
                                spare_blocks=3, poison=True)
    q, kc, vc, table, lens = fa_inputs.make_paged(w)
    q, kc, vc = q.numpy(), kc.numpy(), vc.numpy()
    out, lse = oracle.paged_decode(q, kc, vc, table, lens, w.scale)
    for b in range(w.B):
        for h in range(w.H):
            o, l = alg.paged_attention_blocked(q[b, h, 0], kc[:, h], vc[:, h], table[b].numpy(),
                                               int(lens[b]), w.scale)
            np.testing.assert_allclose(o, out[b, h], rtol=0, atol=1e-12)
            if math.isinf(l):
                assert lse[b, h] == l
            else:
                assert abs(l - lse[b, h]) < 1e-12


def test_planted_mistake_is_caught(monkeypatch):
    """Taking the last block whole (ignoring the length) must fail the
    ragged-length pin: with NaN past the end the output turns NaN."""
    q, k, v = contiguous_case(seed=11)
    kc, table = to_paged(k, 8)
    vc, _ = to_paged(v, 8)
    kc = kc.copy()
    kc[table[0, -1], :, 70 - 8 * (table.shape[1] - 1):] = np.nan

    def whole_blocks(row, seq_len, block_size, num_blocks):
        nb = -(-int(seq_len) // block_size)
        blks = np.repeat(np.asarray(row[:nb], dtype=np.int64), block_size)
        offs = np.tile(np.arange(block_size), nb)
        return blks, offs
    monkeypatch.setattr(oracle, "paged_gather_index", whole_blocks)
    out, _ = oracle.paged_decode(q, kc, vc, table, np.full(3, 70), 0.2)
    assert np.isnan(out[0]).any()


def test_generator_recipe():
    w = fa_inputs.PAGED_WORKLOADS["paged_mixed_f16_b6h4_len1000_d64_bs16_split8"]
    q, kc, vc, table, lens = fa_inputs.make_paged(w)
    assert lens.tolist()[:5] == [0, 1, 15, 17, 1000]
    assert table.dtype == fa_inputs.torch.int32 and lens.dtype == fa_inputs.torch.int32
    mapped = table[table >= 0]
    assert mapped.unique().numel() == mapped.numel()          # no block shared
    assert int(mapped.max()) < kc.shape[0]
    # every row a sequence reads is finite, every other row is NaN
    finite = 0
    for b in range(w.B):
        blks, offs = oracle.paged_gather_index(table[b].numpy(), int(lens[b]), w.block_size, kc.shape[0])
        sel = kc[fa_inputs.torch.from_numpy(blks), :, fa_inputs.torch.from_numpy(offs)]
        assert fa_inputs.torch.isfinite(sel.float()).all()
        finite += blks.size
    assert int((~kc.float().isnan().any(-1)).sum()) == finite * w.H
    a = fa_inputs.make_paged(w)
    assert all(fa_inputs.torch.equal(x.view(-1).float().nan_to_num(7.0), y.view(-1).float().nan_to_num(7.0))
               for x, y in zip(a, (q, kc, vc, table, lens)))
