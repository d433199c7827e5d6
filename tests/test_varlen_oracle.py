"""Pins of the variable-length oracle (``oracle.varlen_attention``) on the CPU.

The varlen oracle cuts each sequence out of the packed tensors and calls the
(pinned) dense ``oracle.attention``; these tests fix the cutting and the
layout from outside:
* sequences of equal length equal the dense [B, H, N, d] call on the same
  numbers (a wrong offset, head or layout transpose breaks it);
* a batch is the concatenation of its sequences: evaluating a sequence alone
  (at offset 0) gives the same bits;
* queries never see keys of another sequence: changing another sequence's
  keys changes nothing;
* causal masking is top-left within each sequence (row 0 of a sequence sees
  exactly its first key);
* an empty query sequence contributes no rows; an empty key sequence gives
  O = 0, LSE = -inf.
"""
import numpy as np
import pytest
import torch

import fa_inputs
import oracle


def packed(B, H, N, d, seed):
    q, k, v = fa_inputs.make_qkv(B, H, N, N, d, "f32", seed)
    pk = lambda t: t.permute(0, 2, 1, 3).reshape(B * N, H, d).contiguous()
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32)
    return (q, k, v), (pk(q), pk(k), pk(v)), cu


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_equal_dense(causal):
    (q, k, v), (pq, pk_, pv), cu = packed(3, 2, 37, 16, 1)
    o, l = oracle.varlen_attention(pq, pk_, pv, cu, cu, 0.25, causal)
    ro, rl = oracle.attention(q, k, v, 0.25, causal)
    np.testing.assert_array_equal(o, ro.transpose(0, 2, 1, 3).reshape(3 * 37, 2, 16))
    np.testing.assert_array_equal(l, rl.transpose(1, 0, 2).reshape(2, 3 * 37))


def test_sequence_alone_gives_same_bits():
    w = fa_inputs.VarlenWorkload("t", 5, 3, 32, "f32", True, 2, 1, 90, same_kv=False)
    q, k, v, cq, ck = fa_inputs.make_varlen(w)
    o, l = oracle.varlen_attention(q, k, v, cq, ck, 0.3, True)
    s = 3
    a, b, c, e = int(cq[s]), int(cq[s + 1]), int(ck[s]), int(ck[s + 1])
    o1, l1 = oracle.varlen_attention(q[a:b], k[c:e], v[c:e], torch.tensor([0, b - a]), torch.tensor([0, e - c]),
                                     0.3, True)
    np.testing.assert_array_equal(o[a:b], o1)
    np.testing.assert_array_equal(l[:, a:b], l1)


def test_other_sequences_keys_do_not_leak():
    w = fa_inputs.VarlenWorkload("t", 4, 2, 16, "f32", False, 3, 10, 40)
    q, k, v, cq, ck = fa_inputs.make_varlen(w)
    o, l = oracle.varlen_attention(q, k, v, cq, ck, 0.3, False)
    k2, v2 = k.clone(), v.clone()
    k2[int(ck[2]):int(ck[3])] += 5.0
    v2[int(ck[2]):int(ck[3])] -= 3.0
    o2, l2 = oracle.varlen_attention(q, k2, v2, cq, ck, 0.3, False)
    for s in (0, 1, 3):
        a, b = int(cq[s]), int(cq[s + 1])
        np.testing.assert_array_equal(o[a:b], o2[a:b])
        np.testing.assert_array_equal(l[:, a:b], l2[:, a:b])
    a, b = int(cq[2]), int(cq[3])
    assert not np.array_equal(o[a:b], o2[a:b])


def test_causal_is_top_left_per_sequence():
    w = fa_inputs.VarlenWorkload("t", 4, 2, 16, "f32", True, 4, 5, 30)
    q, k, v, cq, ck = fa_inputs.make_varlen(w)
    o, l = oracle.varlen_attention(q, k, v, cq, ck, 0.3, True)
    for s in range(4):
        a, c = int(cq[s]), int(ck[s])
        np.testing.assert_array_equal(o[a], v[c].double().numpy())     # only the sequence's first key
        np.testing.assert_allclose(l[:, a], 0.3 * (q[a].double() * k[c].double()).sum(-1).numpy(), atol=1e-12)


def test_empty_sequences():
    w = fa_inputs.VARLEN_WORKLOADS["varlen_mixed_f16_s9h4_len0to700_d64"]
    q, k, v, cq, ck = fa_inputs.make_varlen(w)
    lq = (cq[1:] - cq[:-1]).tolist()
    assert lq[:6] == [0, 1, 127, 128, 129, 700]
    o, l = oracle.varlen_attention(q, k, v, cq, ck, w.scale, True)
    assert np.isfinite(o).all()                  # every row is covered
    # a sequence with queries but no keys: O = 0, LSE = -inf
    cq2 = torch.tensor([0, 3, 5], dtype=torch.int32)
    ck2 = torch.tensor([0, 0, 4], dtype=torch.int32)
    o2, l2 = oracle.varlen_attention(q[:5], k[:4], v[:4], cq2, ck2, 0.3, False)
    assert (o2[:3] == 0).all() and np.isneginf(l2[:, :3]).all()
    assert np.isfinite(l2[:, 3:]).all()


def test_selected_rows_match_full():
    w = fa_inputs.VarlenWorkload("t", 3, 2, 16, "f32", True, 5, 20, 60)
    q, k, v, cq, ck = fa_inputs.make_varlen(w)
    full = oracle.varlen_attention(q, k, v, cq, ck, 0.3, True)
    part = oracle.varlen_attention(q, k, v, cq, ck, 0.3, True, rows={1: [0, 5, int(cq[2] - cq[1]) - 1]})
    a = int(cq[1])
    for i in (0, 5, int(cq[2] - cq[1]) - 1):
        np.testing.assert_array_equal(part[0][a + i], full[0][a + i])
        np.testing.assert_array_equal(part[1][:, a + i], full[1][:, a + i])
