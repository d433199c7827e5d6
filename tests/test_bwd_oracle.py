"""Pins of the backward oracle (``oracle.attention_bwd``) on the CPU.

None compares the oracle with itself:
* torch fp64 autograd of softmax(scale Q K^T + mask) V (a library routine);
* central finite differences of the loss sum(dO * O) through the forward
  oracle, on inputs quantised so that the perturbed values are exact;
* closed forms and invariants: one key gives dQ = dK = 0 and dV = dO;
  the dK rows of a head sum to 0 and the dV rows to the sum of the dO rows
  (the rows of P sum to 1 and those of dS to 0); dQ and dK do not change
  when one vector is added to every key;
* the pages' two-kernel blocked backward (recomputed P from the saved LSE,
  D from the pre-pass) for several block sizes, ragged and causal;
* the block-local rowsum of the first page's block listing differs once a
  row spans more than one K/V block (and agrees when it does not).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import algorithms as alg


def rand(shape, seed, quant=None):
    x = np.random.default_rng(seed).standard_normal(shape)
    if quant:
        x = np.round(x * quant) / quant
    return x.astype(np.float32)


def torch_grads(q, k, v, g, scale, causal):
    Q, K, V = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    S = scale * Q @ K.transpose(-1, -2)
    if causal:
        Nq, Nk = S.shape[-2:]
        vis = torch.ones(Nq, Nk, dtype=torch.bool).tril()
        S = S.masked_fill(~vis, float("-inf"))
    O = torch.softmax(S, -1) @ V
    O.backward(torch.tensor(g, dtype=torch.float64))
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("B,H,Nq,Nk,d", [(1, 2, 5, 7, 4), (2, 1, 33, 33, 16), (1, 1, 40, 17, 8), (1, 3, 1, 9, 32)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd(B, H, Nq, Nk, d, causal):
    q, k, v, g = (rand(s, i) for i, s in enumerate([(B, H, Nq, d), (B, H, Nk, d), (B, H, Nk, d), (B, H, Nq, d)]))
    scale = 1.0 / np.sqrt(d)
    got = oracle.attention_bwd(q, k, v, g, scale, causal)
    ref = torch_grads(q, k, v, g, scale, causal)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    # values on a 1/64 grid, perturbed by 2^-12: every perturbed value is an exact float32
    B, H, Nq, Nk, d = 1, 1, 4, 5, 3
    q, k, v, g = (rand(s, 10 + i, quant=64) for i, s in
                  enumerate([(B, H, Nq, d), (B, H, Nk, d), (B, H, Nk, d), (B, H, Nq, d)]))
    scale = 0.7
    h = 2.0 ** -12

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, scale, causal)
        return float((o * g.astype(np.float64)).sum())

    dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        base = [q, k, v]
        for idx in np.ndindex(base[which].shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += np.float32(h)
            minus[which][idx] -= np.float32(h)
            assert float(plus[which][idx]) - float(base[which][idx]) == h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (which, idx, fd, grad[idx])


def test_single_key_closed_form():
    q, k, v, g = rand((2, 2, 1, 8), 1), rand((2, 2, 1, 8), 2), rand((2, 2, 1, 8), 3), rand((2, 2, 1, 8), 4)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.3, False)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_array_equal(dv, g.astype(np.float64))


@pytest.mark.parametrize("causal", [False, True])
def test_column_sums(causal):
    q, k, v, g = rand((1, 2, 50, 16), 5), rand((1, 2, 60, 16), 6), rand((1, 2, 60, 16), 7), rand((1, 2, 50, 16), 8)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.25, causal)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), g.astype(np.float64).sum(axis=2), atol=1e-12)


def test_key_translation_invariance():
    q, k, v, g = rand((1, 1, 20, 8), 9), rand((1, 1, 20, 8), 10), rand((1, 1, 20, 8), 11), rand((1, 1, 20, 8), 12)
    shift = np.float32(0.5) * rand((8,), 13, quant=4)
    k2 = (k + shift).astype(np.float32)
    a = oracle.attention_bwd(q, k, v, g, 0.35, True)
    b = oracle.attention_bwd(q, k2, v, g, 0.35, True)
    # k2 rounds k + shift to float32; the gradients move only by that rounding
    np.testing.assert_allclose(a[0], b[0], atol=1e-5)
    np.testing.assert_allclose(a[1], b[1], atol=1e-5)
    np.testing.assert_allclose(a[2], b[2], atol=1e-5)


@pytest.mark.parametrize("Br,Bc", [(1, 1), (3, 5), (16, 16), (64, 32)])
@pytest.mark.parametrize("causal", [False, True])
def test_blocked_backward_matches(Br, Bc, causal):
    Nq, Nk, d = 37, 45, 8
    q, k, v, g = rand((1, 1, Nq, d), 20), rand((1, 1, Nk, d), 21), rand((1, 1, Nk, d), 22), rand((1, 1, Nq, d), 23)
    scale = 0.4
    o, lse = oracle.attention(q, k, v, scale, causal)
    ref = oracle.attention_bwd(q, k, v, g, scale, causal)
    got = alg.blocked_backward(q[0, 0], k[0, 0], v[0, 0], o[0, 0], g[0, 0], lse[0, 0], Br, Bc, scale, causal)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b[0, 0], rtol=0, atol=1e-12)


def test_delta_is_rowsum_of_do_times_o():
    q, k, v, g = rand((1, 2, 30, 8), 30), rand((1, 2, 30, 8), 31), rand((1, 2, 30, 8), 32), rand((1, 2, 30, 8), 33)
    o, _ = oracle.attention(q, k, v, 0.3, True)
    *_, delta = oracle.attention_bwd(q, k, v, g, 0.3, True, with_delta=True)
    np.testing.assert_allclose(delta, (o * g.astype(np.float64)).sum(-1), atol=1e-13)


def test_blocklocal_rowsum_is_wrong_across_blocks():
    Nq, Nk, d = 16, 24, 8
    q, k, v, g = rand((1, 1, Nq, d), 40), rand((1, 1, Nk, d), 41), rand((1, 1, Nk, d), 42), rand((1, 1, Nq, d), 43)
    o, lse = oracle.attention(q, k, v, 0.5, False)
    ref = oracle.attention_bwd(q, k, v, g, 0.5, False)
    args = (q[0, 0], k[0, 0], v[0, 0], o[0, 0], g[0, 0], lse[0, 0])
    one_block = alg.blocked_backward(*args, 8, Nk, 0.5, blocklocal_rowsum=True)
    for a, b in zip(one_block, ref):
        np.testing.assert_allclose(a, b[0, 0], atol=1e-12)
    split = alg.blocked_backward(*args, 8, 8, 0.5, blocklocal_rowsum=True)
    assert np.abs(split[0] - ref[0][0, 0]).max() > 1e-3       # dQ is wrong
    assert np.abs(split[1] - ref[1][0, 0]).max() > 1e-3       # dK is wrong
    np.testing.assert_allclose(split[2], ref[2][0, 0], atol=1e-12)   # dV does not use dS


def test_selected_rows_match_full():
    q, k, v, g = rand((2, 2, 40, 16), 50), rand((2, 2, 35, 16), 51), rand((2, 2, 35, 16), 52), rand((2, 2, 40, 16), 53)
    full = oracle.attention_bwd(q, k, v, g, 0.25, True)
    heads, qi, ki = np.array([3, 0]), np.array([0, 39, 17]), np.array([34, 5])
    part = oracle.attention_bwd(q, k, v, g, 0.25, True, heads=heads, q_idx=qi, k_idx=ki)
    for f, p, idx in zip(full, part, (qi, ki, ki)):
        f = f.reshape(4, -1, 16)
        np.testing.assert_array_equal(p, f[heads][:, idx])
