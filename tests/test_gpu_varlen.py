"""GPU parity of the packed variable-length forward (``fa_fwd_varlen``)
against the fp64 oracle (``oracle.varlen_attention``: each sequence on its
own), through the C ABI.

Tolerances are those of the dense 16-bit forward (max |dO| <= 2e-2, mean
|dO| <= 2e-3, max |dLSE| <= 1e-3).  A query whose sequence has no key must
give exactly O = 0 and LSE = -inf.  With every sequence of one length the
packed launch must equal the dense launch bit for bit (same tiles, same
arithmetic, other addressing).
"""
import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from parity_util import compare, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import io_aware_amd
    return io_aware_amd


def run_varlen(fa, w, seqs=None, rows=None):
    note("case " + w.name)
    q, k, v, cq, ck = fa_inputs.make_varlen(w)
    out, lse = fa.fa_fwd_varlen(*to_dev(q, k, v, cq, ck), scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.varlen_attention(q, k, v, cq, ck, w.scale, w.causal, seqs=seqs, rows=rows)
    have = ~np.isnan(ref_l[0])                      # rows the oracle computed
    empty = np.isneginf(ref_l[0]) & have
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    if empty.any():
        assert (o[empty] == 0).all(), w.name + ": O of a query without keys is not 0"
        assert np.isneginf(l[:, empty]).all(), w.name + ": LSE of a query without keys is not -inf"
    keep = have & ~empty
    compare(torch.from_numpy(o[keep]), torch.from_numpy(np.ascontiguousarray(l[:, keep])), ref_o[keep],
            ref_l[:, keep], w.dtype, w.name)
    return out, lse


def test_mixed_lengths_with_empty_sequences(fa):
    run_varlen(fa, fa_inputs.VARLEN_WORKLOADS["varlen_mixed_f16_s9h4_len0to700_d64"])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dims_types_masks(fa, dtype, d, causal):
    w = fa_inputs.VarlenWorkload("varlen %s d%d causal=%d" % (dtype, d, causal), 7, 3, d, dtype, causal,
                                 1100 + d + causal, 1, 400, edge=True, same_kv=not causal)
    run_varlen(fa, w)


def test_full_size_workload_sampled(fa):
    w = fa_inputs.VARLEN_WORKLOADS["varlen_causal_bf16_s16h16_len256to8192_d128"]
    q, k, v, cq, ck = fa_inputs.make_varlen(w)
    lens = (cq[1:] - cq[:-1]).tolist()
    order = np.argsort(lens)
    seqs = [int(order[0]), int(order[len(lens) // 2]), int(order[-1])]
    rng = np.random.default_rng(7)
    rows = {}
    for s in seqs:
        n = lens[s]
        rows[s] = np.unique(np.r_[0, 1, 127, 128, n - 1, rng.integers(0, n, 60)]).clip(0, n - 1)
    out, lse = run_varlen(fa, w, seqs=seqs, rows=rows)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_dense_bitwise(fa, causal):
    B, H, N, d = 4, 8, 1000, 128
    q, k, v = fa_inputs.make_qkv(B, H, N, N, d, "bf16", 1200)
    qd, kd, vd = to_dev(q, k, v)
    o1, l1 = fa.fa_fwd(qd, kd, vd, causal=causal)
    pack = lambda t: t.permute(0, 2, 1, 3).reshape(B * N, H, d).contiguous()
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device=qd.device)
    o2, l2 = fa.fa_fwd_varlen(pack(qd), pack(kd), pack(vd), cu, cu, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(pack(o1), o2)
    assert torch.equal(l1.permute(1, 0, 2).reshape(H, B * N), l2)
