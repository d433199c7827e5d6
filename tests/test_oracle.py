"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check is a brute-force
evaluation at 50 digits, a library routine, a closed form, an invariant, or
an independently written algorithm from the pages that is proved equal to
the definition.  A planted mistake (a blocked forward without the rescale)
must fail them.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle
from oracle import algorithms as alg

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_qkv(B, H, Nq, Nk, d, seed, q_sigma=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, H, Nq, d)) * q_sigma).astype(np.float32)
    k = rng.standard_normal((B, H, Nk, d)).astype(np.float32)
    v = rng.standard_normal((B, H, Nk, d)).astype(np.float32)
    return q, k, v


def torch_reference_f64(q, k, v, scale, causal):
    """softmax(scale * Q K^T + mask) V and logsumexp with torch's fp64 library
    routines (the reference the Triton page's test uses, in fp64)."""
    Q, K, V = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (q, k, v))
    S = torch.matmul(Q, K.transpose(-1, -2)) * scale
    if causal:
        Nq, Nk = S.shape[-2], S.shape[-1]
        mask = torch.arange(Nk)[None, :] > torch.arange(Nq)[:, None]
        S = S.masked_fill(mask, float("-inf"))
    P = torch.softmax(S, dim=-1)
    return (P @ V).numpy(), torch.logsumexp(S, dim=-1).numpy()


# ---------------------------------------------------------------------------
# 1-D online softmax = three-pass softmax (proved identity)
# ---------------------------------------------------------------------------

ADVERSARIAL = {
    "random": np.random.default_rng(1).standard_normal(97) * 3,
    "increasing": np.arange(50, dtype=np.float64) * 0.7,       # max moves every step
    "decreasing": -np.arange(50, dtype=np.float64) * 0.7,
    "ties": np.array([2.0, 2.0, 2.0, -1.0, 2.0]),
    "huge": np.array([1000.0, -1000.0, 999.0, 1000.0, 0.0]),     # naive exp overflows
    "tiny": np.array([-1000.0, -1001.0, -999.5]),                  # naive exp underflows
    "with_neg_inf": np.array([-np.inf, 0.5, -np.inf, 3.0, -2.0]),
    "single": np.array([4.2]),
}


@pytest.mark.parametrize("name", sorted(ADVERSARIAL))
def test_online_softmax_equals_three_pass(name):
    x = ADVERSARIAL[name]
    ref = alg.softmax_three_pass(x)
    got = alg.online_softmax(x)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-300)
    # the one-pass statistics equal the statistics against the final max
    m, l = alg.online_softmax_stats(x)
    finite = x[np.isfinite(x)]
    assert m == finite.max()
    assert math.isclose(l, float(np.exp(finite - finite.max()).sum()), rel_tol=1e-14)


@pytest.mark.parametrize("name", sorted(ADVERSARIAL))
@pytest.mark.parametrize("block", [1, 2, 7, 64])
def test_block_statistics_equal_one_pass(name, block):
    x = ADVERSARIAL[name]
    m1, l1 = alg.online_softmax_stats(x)
    m2, l2 = alg.blockwise_softmax_stats(x, block)
    assert m1 == m2
    assert math.isclose(l1, l2, rel_tol=1e-14)


def test_three_pass_softmax_matches_library():
    import scipy.special
    for name, x in ADVERSARIAL.items():
        np.testing.assert_allclose(alg.softmax_three_pass(x), scipy.special.softmax(x),
                                   rtol=1e-13, atol=1e-300, err_msg=name)


def test_hand_worked_softmax():
    # scores 0 and ln 3: weights exactly 1/4 and 3/4; logsumexp = ln 4
    x = np.array([0.0, math.log(3.0)])
    np.testing.assert_allclose(alg.softmax_three_pass(x), [0.25, 0.75], rtol=1e-15)
    m, l = alg.online_softmax_stats(x)
    assert math.isclose(m + math.log(l), math.log(4.0), rel_tol=1e-15)


# ---------------------------------------------------------------------------
# The C oracle against brute force and a library routine
# ---------------------------------------------------------------------------

def mp_attention(q, k, v, scale, causal, dps=50):
    """O and LSE for one head by brute force in 50-digit arithmetic."""
    mpmath.mp.dps = dps
    Nq, d = q.shape
    Nk = k.shape[0]
    out = np.zeros((Nq, d))
    lse = np.zeros(Nq)
    sc = mpmath.mpf(float(scale))
    for i in range(Nq):
        vis = range(Nk) if not causal else range(min(i + 1, Nk))
        s = [sc * mpmath.fsum(mpmath.mpf(float(q[i, t])) * mpmath.mpf(float(k[j, t]))
                              for t in range(d)) for j in vis]
        e = [mpmath.exp(x) for x in s]
        z = mpmath.fsum(e)
        for t in range(d):
            out[i, t] = float(mpmath.fsum(e[n] * mpmath.mpf(float(v[j, t]))
                                          for n, j in enumerate(vis)) / z)
        lse[i] = float(mpmath.log(z))
    return out, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk,d,sigma", [(5, 7, 4, 1.0), (8, 8, 8, 1.0), (6, 3, 5, 8.0), (1, 8, 8, 30.0)])
def test_oracle_matches_mpmath(causal, Nq, Nk, d, sigma):
    q, k, v = rand_qkv(1, 1, Nq, Nk, d, seed=Nq * 100 + Nk, q_sigma=sigma)
    scale = float(np.float32(1 / math.sqrt(d)))
    out, lse = oracle.attention(q, k, v, scale, causal)
    ref_o, ref_l = mp_attention(q[0, 0], k[0, 0], v[0, 0], scale, causal)
    np.testing.assert_allclose(out[0, 0], ref_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], ref_l, rtol=1e-14, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [-0.35, -3.0, 0.0])
def test_oracle_matches_mpmath_at_negative_and_zero_scale(causal, scale):
    # the caller's scale may be any finite value ("08. Triton Flash
    # Attention": the kernel takes sm_scale as an argument)
    q, k, v = rand_qkv(1, 1, 6, 7, 5, seed=611, q_sigma=2.0)
    out, lse = oracle.attention(q, k, v, scale, causal)
    ref_o, ref_l = mp_attention(q[0, 0], k[0, 0], v[0, 0], scale, causal)
    np.testing.assert_allclose(out[0, 0], ref_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], ref_l, rtol=1e-14, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_gives_mean_of_visible_values(causal):
    # every visible score is 0, so P is uniform over the visible keys:
    # O_i = mean of the visible v_j and LSE_i = ln |J_i|
    q, k, v = rand_qkv(1, 2, 20, 25, 8, seed=612, q_sigma=5.0)
    out, lse = oracle.attention(q, k, v, 0.0, causal)
    v64 = v.astype(np.float64)
    for i in range(20):
        n = (i + 1) if causal else 25
        np.testing.assert_allclose(out[0, :, i], v64[0, :, :n].mean(axis=1), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, :, i], math.log(n), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Nq,Nk,d", [(1, 1, 256, 256, 64), (2, 3, 100, 100, 64), (1, 2, 37, 61, 32),
                                         (1, 1, 70, 33, 128)])
def test_oracle_matches_torch_fp64(causal, B, H, Nq, Nk, d):
    q, k, v = rand_qkv(B, H, Nq, Nk, d, seed=B * 7 + Nq)
    scale = float(np.float32(1 / math.sqrt(d)))
    out, lse = oracle.attention(q, k, v, scale, causal)
    ref_o, ref_l = torch_reference_f64(q, k, v, scale, causal)
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms and invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_constant_value_rows_give_that_constant(causal):
    q, k, _ = rand_qkv(2, 2, 50, 64, 16, seed=3, q_sigma=4.0)
    c = np.random.default_rng(4).standard_normal(16).astype(np.float32)
    v = np.broadcast_to(c, k.shape).copy()
    out, _ = oracle.attention(q, k, v, 0.25, causal)
    np.testing.assert_allclose(out, np.broadcast_to(c.astype(np.float64), out.shape),
                               rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_every_row_of_p_sums_to_one(causal):
    # with a value column of ones, that output column is sum_j P_ij
    q, k, v = rand_qkv(1, 2, 40, 40, 8, seed=5, q_sigma=6.0)
    v[..., 3] = 1.0
    out, _ = oracle.attention(q, k, v, 0.5, causal)
    np.testing.assert_allclose(out[..., 3], 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_values(causal):
    q, k, v = rand_qkv(1, 2, 30, 30, 8, seed=6)
    k[:] = k[:, :, :1, :]                      # every key equal to key 0
    scale = 0.35
    out, lse = oracle.attention(q, k, v, scale, causal)
    v64 = v.astype(np.float64)
    for h in range(2):
        for i in range(30):
            n = (i + 1) if causal else 30
            np.testing.assert_allclose(out[0, h, i], v64[0, h, :n].mean(axis=0), rtol=0, atol=1e-14)
            s = scale * float(np.dot(q[0, h, i].astype(np.float64), k[0, h, 0].astype(np.float64)))
            assert math.isclose(lse[0, h, i], s + math.log(n), rel_tol=0, abs_tol=1e-13)


def test_causal_first_row_is_first_value():
    q, k, v = rand_qkv(2, 3, 20, 20, 16, seed=7, q_sigma=8.0)
    scale = 0.25
    out, lse = oracle.attention(q, k, v, scale, True)
    np.testing.assert_array_equal(out[:, :, 0], v[:, :, 0].astype(np.float64))
    s00 = scale * np.einsum("bhd,bhd->bh", q[:, :, 0].astype(np.float64), k[:, :, 0].astype(np.float64))
    np.testing.assert_allclose(lse[:, :, 0], s00, rtol=0, atol=1e-13)


def test_key_value_permutation_equivariance():
    q, k, v = rand_qkv(1, 2, 33, 50, 16, seed=8)
    perm = np.random.default_rng(9).permutation(50)
    out1, lse1 = oracle.attention(q, k, v, 0.25, False)
    out2, lse2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.25, False)
    np.testing.assert_allclose(out2, out1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse1, rtol=0, atol=1e-13)


def test_large_scores_do_not_overflow():
    q, k, v = rand_qkv(1, 1, 16, 16, 8, seed=10, q_sigma=400.0)   # scores in the thousands
    out, lse = oracle.attention(q, k, v, 1.0, False)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ref_o, ref_l = torch_reference_f64(q, k, v, 1.0, False)
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_l, rtol=1e-14)


# ---------------------------------------------------------------------------
# The pages' blocked algorithms equal the definition
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Br,Bc", [(1, 1), (3, 16), (16, 3), (64, 64), (16, 64), (64, 16)])
@pytest.mark.parametrize("Nq,Nk", [(100, 100), (37, 70), (70, 37)])
def test_blocked_forms_equal_oracle(causal, Br, Bc, Nq, Nk):
    q, k, v = rand_qkv(1, 1, Nq, Nk, 8, seed=Br * 1000 + Bc + Nq, q_sigma=3.0)
    out, lse = oracle.attention(q, k, v, 0.3, causal)
    for normalized in (False, True):
        o2, l2 = alg.blocked_attention_bhsd(q, k, v, Br, Bc, 0.3, causal, normalized=normalized)
        np.testing.assert_allclose(o2, out, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-12)


def test_missing_rescale_is_detected():
    """A blocked forward without exp(m_old - m_new) fails on inputs shaped like
    the long-sequence workload (q scaled by 8): the pins catch a rescale bug."""
    q, k, v = rand_qkv(1, 1, 128, 512, 128, seed=11, q_sigma=8.0)
    scale = float(np.float32(1 / math.sqrt(128)))
    out, lse = oracle.attention(q, k, v, scale, False)
    good, _ = alg.blocked_attention(q[0, 0], k[0, 0], v[0, 0], 64, 64, scale, False, rescale=True)
    bad, _ = alg.blocked_attention(q[0, 0], k[0, 0], v[0, 0], 64, 64, scale, False, rescale=False)
    np.testing.assert_allclose(good, out[0, 0], rtol=0, atol=1e-12)
    assert np.abs(bad - out[0, 0]).max() > 0.5          # far outside any tolerance


# ---------------------------------------------------------------------------
# Split-KV partials and their merge
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("Nk,splits", [(8192, 32), (1000, 7), (100, 32), (5, 8), (256, 1)])
def test_split_merge_equals_unsplit(Nk, splits):
    q, k, v = rand_qkv(1, 1, 1, Nk, 16, seed=Nk + splits, q_sigma=2.0)
    out, lse = oracle.attention(q, k, v, 0.25, False)
    parts = alg.split_partials(q[0, 0, 0], k[0, 0], v[0, 0], 0.25, splits)
    o_seq, lse_seq = alg.merge_partials(parts)
    np.testing.assert_allclose(o_seq, out[0, 0, 0], rtol=0, atol=1e-12)
    assert math.isclose(lse_seq, lse[0, 0, 0], abs_tol=1e-12)
    lse_c = [p["m"] + math.log(p["l"]) if p["l"] > 0 else -math.inf for p in parts]
    o_t = [p["o"] / p["l"] if p["l"] > 0 else np.zeros(16) for p in parts]
    o_c, lse_cmb = alg.combine_lse(lse_c, o_t)
    np.testing.assert_allclose(o_c, out[0, 0, 0], rtol=0, atol=1e-12)
    assert math.isclose(lse_cmb, lse[0, 0, 0], abs_tol=1e-12)


def _parts_from_scores(chunks):
    parts = []
    for s, vv in chunks:
        p = np.exp(s - s.max())
        parts.append({"m": float(s.max()), "l": float(p.sum()), "o": p @ vv})
    return parts


def test_fixed_reference_merge_only_fails_by_overflow():
    """The first page's faulty merge keeps chunk 1's max as a fixed reference
    and weighs chunk j by exp(m_j - m_1).  In exact arithmetic that is the
    same merge (every chunk is moved to one common reference), so with the
    page's maxima 10 and 20 it agrees with the online merge; it breaks only
    when exp(m_j - m_1) overflows, which the online merge never risks."""
    with open(os.path.join(GOLDEN, "merge_demo.json")) as f:
        demo = json.load(f)
    m1, m2 = demo["block_maxima"]
    v1 = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    v2 = np.array([[2.0, -1.0], [0.5, 0.5]])
    s1 = np.array([m1, m1 - 1.0, m1 - 2.5])
    s2 = np.array([m2, m2 - 0.5])
    parts = _parts_from_scores([(s1, v1), (s2, v2)])
    truth = alg.softmax_three_pass(np.concatenate([s1, s2])) @ np.vstack([v1, v2])
    good, _ = alg.merge_partials(parts)
    np.testing.assert_allclose(good, truth, rtol=1e-14)
    # the faulty merge weighs chunk 2 by exp(m2 - m1) = exp(10) ~ 22026 ...
    factor = math.exp(m2 - m1)
    assert math.isclose(factor, demo["wrong_merge_weight_of_block2"],
                        rel_tol=demo["wrong_merge_weight_of_block2_rel_tol"])
    bad = alg.wrong_merge(parts)
    l_wrong = parts[0]["l"] + parts[1]["l"] * factor
    np.testing.assert_allclose(bad, (parts[0]["o"] + parts[1]["o"] * factor) / l_wrong, rtol=1e-14)
    # ... which is the right relative weight, so the result agrees
    np.testing.assert_allclose(bad, truth, rtol=1e-13)
    # chunk maxima 10 and 1000: exp(990) overflows double, the faulty merge
    # returns inf/inf, the online merge stays exact
    s3 = np.array([1000.0, 999.0])
    parts = _parts_from_scores([(s1, v1), (s3, v2)])
    truth = alg.softmax_three_pass(np.concatenate([s1, s3])) @ np.vstack([v1, v2])
    np.testing.assert_allclose(alg.merge_partials(parts)[0], truth, rtol=1e-14)
    with np.errstate(over="ignore", invalid="ignore"):
        try:
            bad = alg.wrong_merge(parts)
        except OverflowError:
            bad = np.full(2, np.nan)
    assert not np.isfinite(bad).all()


# ---------------------------------------------------------------------------
# The oracle's interface
# ---------------------------------------------------------------------------

def test_row_subset_equals_full():
    q, k, v = rand_qkv(2, 3, 77, 90, 32, seed=12)
    full_o, full_l = oracle.attention(q, k, v, 0.2, True)
    rows = np.array([0, 5, 76, 77, 300, 2 * 3 * 77 - 1])
    o, l = oracle.attention(q, k, v, 0.2, True, rows=rows)
    np.testing.assert_array_equal(o, full_o.reshape(-1, 32)[rows])
    np.testing.assert_array_equal(l, full_l.reshape(-1)[rows])


def test_bad_rows_raise():
    q, k, v = rand_qkv(1, 1, 4, 4, 4, seed=13)
    with pytest.raises(RuntimeError):
        oracle.attention(q, k, v, 1.0, False, rows=[0, 4])


def test_thread_count_does_not_change_results():
    q, k, v = rand_qkv(1, 4, 64, 64, 16, seed=14)
    a = oracle.attention(q, k, v, 0.25, True, threads=1)
    b = oracle.attention(q, k, v, 0.25, True, threads=4)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
