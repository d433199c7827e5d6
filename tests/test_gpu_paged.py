"""GPU parity of the paged-cache decode (``fa_fwd_paged_decode``) against the
fp64 oracle (``oracle.paged_decode``: the mapped keys gathered in logical
order, then exact attention), on the same seeded inputs, through the C ABI.

Tolerances are those of the other fp16 / bf16 paths (max |dO| <= 2e-2, mean
|dO| <= 2e-3, max |dLSE| <= 1e-3).  A sequence with no key must give O = 0
and LSE = -inf exactly.  The full-size workload (the launch bench.py times)
is compared on a sample of whole sequences, and in full against the
contiguous split-KV path, which it must match bit for bit when the table
maps every sequence's keys in order.
"""
import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from parity_util import DEV, compare, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import io_aware_amd
    return io_aware_amd


def run_paged(fa, q, kc, vc, table, lens, S, scale, dtype, label, seqs=None):
    note("case " + label)
    out, lse = fa.fa_fwd_paged_decode(*to_dev(q, kc, vc, table, lens), S, scale=scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.paged_decode(q, kc, vc, table, lens, scale, seqs=seqs)
    sel = list(range(q.shape[0])) if seqs is None else list(seqs)
    o = out[sel, :, 0].float().cpu()
    l = lse[sel].cpu()
    empty = np.isneginf(ref_l)
    if empty.any():
        e = torch.from_numpy(empty)
        assert (o[e] == 0).all(), label + ": O of an empty sequence is not 0"
        assert torch.isneginf(l[e]).all(), label + ": LSE of an empty sequence is not -inf"
    keep = torch.from_numpy(~empty)
    if keep.any():
        compare(o[keep], l[keep], ref_o[~empty], ref_l[~empty], dtype, label)
    return out, lse


def test_full_size_workload_sampled_sequences(fa):
    w = fa_inputs.PAGED_WORKLOADS["paged_decode_bf16_b16h32_len8192_d128_bs16_split32"]
    q, kc, vc, table, lens = fa_inputs.make_paged(w)
    out, lse = run_paged(fa, q, kc, vc, table, lens, w.num_splits, w.scale, w.dtype, w.name, seqs=[0, 7, 15])
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_full_size_identity_table_matches_contiguous_splitkv(fa):
    """With sequence b's logical block j at physical block b*nb + j and a
    head-major cache, the paged kernel reads the same keys in the same
    order and chunking as the contiguous split-KV path: bitwise equal."""
    w = fa_inputs.WORKLOADS["decode_bf16_b16h32_nk8192_d128_split32"]
    note("case identity table " + w.name)
    q, k, v = fa_inputs.make_workload(w)
    B, H, N, d = k.shape
    bs = 16
    nb = N // bs
    # [B, H, N, d] -> [B*nb, H, bs, d]
    kc = k.reshape(B, H, nb, bs, d).permute(0, 2, 1, 3, 4).reshape(B * nb, H, bs, d).contiguous()
    vc = v.reshape(B, H, nb, bs, d).permute(0, 2, 1, 3, 4).reshape(B * nb, H, bs, d).contiguous()
    table = torch.arange(B * nb, dtype=torch.int32).reshape(B, nb)
    lens = torch.full((B,), N, dtype=torch.int32)
    qd, kd, vd, kcd, vcd, td, ld = to_dev(q, k, v, kc, vc, table, lens)
    o1, l1 = fa.fa_fwd_splitkv(qd, kd, vd, w.num_splits, scale=w.scale)
    o2, l2 = fa.fa_fwd_paged_decode(qd, kcd, vcd, td, ld, w.num_splits, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1.reshape(B, H), l2)


def test_mixed_lengths_holes_and_poison(fa):
    w = fa_inputs.PAGED_WORKLOADS["paged_mixed_f16_b6h4_len1000_d64_bs16_split8"]
    q, kc, vc, table, lens = fa_inputs.make_paged(w)
    run_paged(fa, q, kc, vc, table, lens, w.num_splits, w.scale, w.dtype, w.name)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("bs,max_len,S", [(1, 97, 5), (16, 700, 16), (64, 1500, 3), (1024, 2100, 64)])
def test_block_sizes_and_dims(fa, dtype, d, bs, max_len, S):
    w = fa_inputs.PagedWorkload("paged %s d%d bs%d len%d S%d" % (dtype, d, bs, max_len, S), 5, 3, d, bs,
                                max_len, dtype, 2000 + d + bs + S, S, lens="mixed", hole_frac=0.15,
                                spare_blocks=2, poison=True)
    q, kc, vc, table, lens = fa_inputs.make_paged(w)
    run_paged(fa, q, kc, vc, table, lens, S, w.scale, dtype, w.name)


def test_out_of_range_entries_are_skipped(fa):
    w = fa_inputs.PagedWorkload("oor", 4, 2, 128, 16, 400, "bf16", 3001, 4, poison=True)
    q, kc, vc, table, lens = fa_inputs.make_paged(w)
    t = table.clone()
    t[0, 3] = kc.shape[0]            # one past the cache
    t[1, 0] = 1 << 30
    t[2, 5] = -2
    run_paged(fa, q, kc, vc, t, lens, 4, w.scale, "bf16", "out-of-range table entries")


def test_lengths_past_the_table_and_negative(fa):
    w = fa_inputs.PagedWorkload("clamp", 3, 2, 64, 16, 160, "bf16", 3002, 3)
    q, kc, vc, table, lens = fa_inputs.make_paged(w)
    l2 = torch.tensor([10 ** 6, -3, 0], dtype=torch.int32)
    run_paged(fa, q, kc, vc, table, l2, 3, w.scale, "bf16", "clamped lengths")


def test_shared_kv_tensor_and_deterministic(fa):
    """The page's single [2, num_blocks, H, block_size, d] cache passes as its
    two halves; repeated calls give identical bits."""
    w = fa_inputs.PagedWorkload("kv2", 4, 4, 128, 32, 900, "bf16", 3003, 8, lens="mixed")
    q, kc, vc, table, lens = fa_inputs.make_paged(w)
    kv = torch.stack([kc, vc]).to(DEV)
    qd, td, ld = to_dev(q, table, lens)
    a = fa.fa_fwd_paged_decode(qd, kv[0], kv[1], td, ld, 8, scale=w.scale)
    b = fa.fa_fwd_paged_decode(qd, kv[0], kv[1], td, ld, 8, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    ref_o, ref_l = oracle.paged_decode(q, kc, vc, table, lens, w.scale)
    keep = ~np.isneginf(ref_l)
    compare(a[0][:, :, 0].cpu()[torch.from_numpy(keep)], a[1].cpu()[torch.from_numpy(keep)],
            ref_o[keep], ref_l[keep], "bf16", "shared kv tensor")
