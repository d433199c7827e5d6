"""Pins of the FP8 oracle (``oracle.fp8``) on the CPU.

* the butterfly transform equals x @ H_d with scipy's Hadamard matrix, and
  applying it twice gives d * x;
* the incoherent transform is orthogonal: it keeps dot products (Q K^T) and
  norms up to float32 rounding, and the same signs must go to Q and K;
* E4M3 rounding equals a brute-force nearest-value search over all 256
  codes with ties to the even code, on every midpoint of the format;
* per-head quantisation maps the largest magnitude to +-448 exactly and
  keeps every value within half a unit in the last place;
* the FP8 attention oracle equals exact attention when the inputs are
  already E4M3 values with amax 448 (the quantisation is then the identity);
* incoherent processing does what the page says it is for: with a few
  large-magnitude channels in Q and K, the error of the quantised scores is
  smaller with the transform than without.
"""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from oracle import fp8


def all_e4m3():
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8.e4m3_values(codes)
    ok = np.isfinite(vals)
    return codes[ok], vals[ok]


@pytest.mark.parametrize("d", [8, 32, 64, 128])
def test_fwht_matches_hadamard_matrix(d):
    x = np.random.default_rng(d).standard_normal((5, d)).astype(np.float32)
    ref = x.astype(np.float64) @ scipy.linalg.hadamard(d)
    np.testing.assert_allclose(fp8.fwht_f32(x), ref, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(fp8.fwht_f32(fp8.fwht_f32(x)), d * x, rtol=1e-5, atol=1e-3)


def test_transform_is_orthogonal():
    rng = np.random.default_rng(1)
    d = 128
    signs = rng.choice([-1.0, 1.0], d).astype(np.float32)
    q = rng.standard_normal((40, d)).astype(np.float32)
    k = rng.standard_normal((30, d)).astype(np.float32)
    qt, kt = fp8.incoherent_transform(q, signs), fp8.incoherent_transform(k, signs)
    np.testing.assert_allclose(qt.astype(np.float64) @ kt.T, q.astype(np.float64) @ k.T, atol=2e-4)
    np.testing.assert_allclose(np.linalg.norm(qt, axis=1), np.linalg.norm(q, axis=1), rtol=1e-5)
    # different signs for Q and K do not preserve the scores
    other = -signs
    other[:64] = signs[:64]
    kx = fp8.incoherent_transform(k, other)
    assert np.abs(qt.astype(np.float64) @ kx.T - q.astype(np.float64) @ k.T).max() > 1.0


def test_e4m3_rounding_is_nearest_even():
    codes, vals = all_e4m3()
    pos = np.sort(np.unique(vals[vals >= 0]))
    mids = (pos[:-1] + pos[1:]) / 2
    probes = np.concatenate([pos, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                             np.nextafter(mids.astype(np.float32), np.float32(1000))]).astype(np.float32)
    probes = np.concatenate([probes, -probes])
    got = fp8.e4m3_values(fp8.to_e4m3_codes(probes))
    for x, g in zip(probes.astype(np.float64), got):
        dist = np.abs(vals - x)
        best = np.flatnonzero(dist == dist.min())
        if best.size > 1:       # a tie: the code with an even mantissa (even code)
            cand = codes[best]
            want = vals[best[np.flatnonzero(cand % 2 == 0)[0]]]
        else:
            want = vals[best[0]]
        assert g == want or (g == 0 and want == 0), (x, g, want)


def test_quantize_heads_bounds():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((2, 3, 50, 16)) * rng.uniform(0.01, 100, (2, 3, 1, 1))).astype(np.float32)
    x[1, 2] = 0.0
    codes, descale = fp8.quantize_heads(x)
    deq = fp8.dequantize(codes, descale)
    amax = np.abs(x).reshape(2, 3, -1).max(-1)
    for b in range(2):
        for h in range(3):
            if amax[b, h] == 0:
                assert (deq[b, h] == 0).all() and descale[b, h] == 1.0
                continue
            assert np.abs(deq[b, h]).max() == pytest.approx(amax[b, h], rel=1e-6)
            # relative error of a normal E4M3 value: at most 2^-4 (half a unit, 3 mantissa bits)
            big = np.abs(x[b, h]) > amax[b, h] * 2.0 ** -6 * 1.01
            rel = np.abs(deq[b, h][big] - x[b, h][big]) / np.abs(x[b, h][big])
            assert rel.max() <= 2.0 ** -4 + 1e-6


def test_identity_quantisation_gives_exact_attention():
    codes, vals = all_e4m3()
    rng = np.random.default_rng(3)
    B, H, N, d = 1, 2, 40, 32
    pick = lambda: rng.choice(vals[np.abs(vals) <= 16], size=(B, H, N, d)).astype(np.float32)
    q, k, v = pick(), pick(), pick()
    for t in (q, k, v):      # amax 448 per head: the scale is 1, codes are the values
        t[:, :, 0, 0] = 448.0
    out, lse, qu = fp8.fp8_attention(q, k, v, 0.1, True)
    ro, rl = oracle.attention(q, k, v, 0.1, True)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)
    assert (qu["dq"] == 1).all() and (qu["dv"] == 1).all()


def test_incoherent_processing_reduces_score_error():
    rng = np.random.default_rng(4)
    B, H, N, d = 1, 2, 256, 128
    q = rng.standard_normal((B, H, N, d)).astype(np.float32)
    k = rng.standard_normal((B, H, N, d)).astype(np.float32)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    q[..., :4] *= 40.0          # a few outlier channels, as activations have
    k[..., :4] *= 40.0
    signs = rng.choice([-1.0, 1.0], d).astype(np.float32)
    exact = q.astype(np.float64) @ k.astype(np.float64).transpose(0, 1, 3, 2)

    def score_err(sg):
        qu = fp8.quantize_qkv(q, k, v, sg)
        qd = fp8.dequantize(qu["q8"], qu["dq"])
        kd = fp8.dequantize(qu["k8"], qu["dk"])
        return np.abs(qd @ kd.transpose(0, 1, 3, 2) - exact).mean()
    plain, incoherent = score_err(None), score_err(signs)
    assert incoherent < 0.5 * plain, (plain, incoherent)
