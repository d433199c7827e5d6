"""GPU parity of the FP8 path against the oracle (``oracle.fp8``), through the
C ABI.

* Quantisation (``fa_quantize_fp8``): the E4M3 codes of Q M, K M and V and
  the descale factors must equal the oracle's bit for bit (the transform and
  the rounding are taken in float32 in the same order on both sides); the
  transposed, permuted V codes are compared through the documented layout.
* Forward (``fa_fwd_fp8``) against exact attention on the same dequantised
  inputs.  The kernel rounds P to E4M3 before P V' (3 mantissa bits) and
  normalises by the sum of the rounded P; the pages give no bound for FP8,
  so the bar comes from the arithmetic: tests/rounding_models.py models
  those rounding points on the CPU (P relative to a held max up to 2^8
  above it, rounded to E4M3; the sum of the rounded P; float32
  accumulation; bf16 output), and on the cases below (the same shapes and
  seeds) gives at most max |dO| = 0.070 and mean |dO| = 3.8e-3, matching
  what the GPU measures (tests/test_models.py recomputes them).  The tests
  allow about 1.7x and 2x that (parity_util):
      max |dO| <= 0.12,  mean |dO| <= 8e-3,  max |dLSE| <= 1e-3.
* End to end against exact attention on the unquantised inputs (q not
  scaled): the model gives mean |dO| of at most 5e-3; the test allows
  mean |dO| <= 1e-2.
"""
import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from oracle import fp8
from parity_util import DEV, FP8_EXACT_MEAN, FP8_LSE, FP8_MAX, FP8_MEAN, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import io_aware_amd
    return io_aware_amd


def up(x):
    return (x + 255) // 256 * 256


def unpack(pack, B, H, Nq, Nk, d):
    """Split a pack (device uint8 tensor) into numpy parts by the documented layout."""
    BH = B * H
    Nkp = (Nk + 63) // 64 * 64
    p = pack.cpu().numpy()
    o_k = up(BH * Nq * d)
    o_v = o_k + up(BH * Nkp * d)
    o_s = o_v + up(BH * d * Nkp)
    q8 = p[:BH * Nq * d].reshape(B, H, Nq, d)
    k8 = p[o_k:o_k + BH * Nkp * d].reshape(B, H, Nkp, d)
    v8t = p[o_v:o_v + BH * d * Nkp].reshape(B, H, d, Nkp)
    desc = p[o_s:o_s + 12 * BH].view(np.float32).reshape(3, B, H)
    # undo the key permutation of V^T: position p = 32g + 16b + r holds key 32b + 8(r/4) + 4g + r%4
    pos = np.arange(Nkp)
    w = pos % 64
    g, b, r = w // 32, (w // 16) % 2, w % 16
    key = pos - w + 32 * b + 8 * (r // 4) + 4 * g + r % 4
    v8 = np.empty((B, H, Nkp, d), dtype=np.uint8)
    v8[:, :, key, :] = v8t.transpose(0, 1, 3, 2)
    return q8, k8, v8, desc


def signs_dev(d, seed):
    return fa_inputs.make_signs(d, seed).to(DEV)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("transform", [False, True])
def test_quantize_bit_exact(fa, dtype, d, transform):
    B, H, Nq, Nk = 2, 3, 200, 333
    note("case quantize %s d%d transform=%d" % (dtype, d, transform))
    q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, dtype, 1300 + d, q_sigma=3.0)
    signs = fa_inputs.make_signs(d, 1300) if transform else None
    pack = fa.fa_quantize_fp8(*to_dev(q, k, v), signs=None if signs is None else signs.to(DEV))
    torch.cuda.synchronize()
    q8, k8, v8, desc = unpack(pack, B, H, Nq, Nk, d)
    ref = fp8.quantize_qkv(q, k, v, None if signs is None else signs.numpy())
    np.testing.assert_array_equal(q8, ref["q8"])
    np.testing.assert_array_equal(k8[:, :, :Nk], ref["k8"])
    np.testing.assert_array_equal(v8[:, :, :Nk], ref["v8"])
    assert (k8[:, :, Nk:] == 0).all() and (v8[:, :, Nk:] == 0).all()
    np.testing.assert_array_equal(desc[0], ref["dq"])
    np.testing.assert_array_equal(desc[1], ref["dk"])
    np.testing.assert_array_equal(desc[2], ref["dv"])


def test_e4m3_rounding_matches_reference(fa):
    # no transform, amax 448: the codes are the rounding of the values themselves
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8.e4m3_values(codes)
    pos = np.sort(np.unique(vals[np.isfinite(vals) & (vals >= 0)]))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(500)),
                           pos.astype(np.float32)])
    # bf16 cannot hold every probe exactly: use the probes that it can
    keep = torch.from_numpy(near).to(torch.bfloat16).float().numpy() == near
    x = np.concatenate([near[keep], -near[keep]]).astype(np.float32)
    d = 64
    n = (x.size + d - 1) // d
    buf = np.zeros(n * d, dtype=np.float32)
    buf[:x.size] = x
    buf[0] = 448.0
    q = torch.from_numpy(buf.reshape(1, 1, n, d)).to(torch.bfloat16)
    pack = fa.fa_quantize_fp8(*to_dev(q, q, q))
    torch.cuda.synchronize()
    q8, _, _, desc = unpack(pack, 1, 1, n, n, d)
    assert desc[0, 0, 0] == 1.0
    np.testing.assert_array_equal(q8.reshape(-1), fp8.to_e4m3_codes(buf))


def run_fp8(fa, B, H, Nq, Nk, d, causal, seed, q_sigma=1.0, transform=True, exact_check=False, label=None):
    label = label or "fp8 B%d H%d Nq%d Nk%d d%d causal=%d t=%d" % (B, H, Nq, Nk, d, causal, transform)
    note("case " + label)
    q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, "bf16", seed, q_sigma)
    signs = fa_inputs.make_signs(d, seed) if transform else None
    scale = fa_inputs.default_scale(d)
    pack = fa.fa_quantize_fp8(*to_dev(q, k, v), signs=None if signs is None else signs.to(DEV))
    out, lse = fa.fa_fwd_fp8(pack, B, H, Nq, Nk, d, scale=scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl, _ = fp8.fp8_attention(q, k, v, scale, causal, signs=None if signs is None else signs.numpy())
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    err, lerr = np.abs(o - ro), np.abs(l - rl)
    note("%s: max|dO|=%.3e mean|dO|=%.3e max|dLSE|=%.3e" % (label, err.max(), err.mean(), lerr.max()))
    assert err.max() <= FP8_MAX and err.mean() <= FP8_MEAN and lerr.max() <= FP8_LSE, label
    if exact_check:
        eo, _ = oracle.attention(q, k, v, scale, causal)
        e2 = np.abs(o - eo)
        note("%s vs exact: max|dO|=%.3e mean|dO|=%.3e" % (label, e2.max(), e2.mean()))
        assert e2.mean() <= FP8_EXACT_MEAN, label
    return out, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_ragged(fa, d, causal):
    run_fp8(fa, 1, 2, 300, 517, d, causal, 1400 + d)
    run_fp8(fa, 2, 1, 129, 64, d, causal, 1401 + d)
    run_fp8(fa, 1, 1, 1, 77, d, causal, 1402 + d)


def test_forward_medium_and_exact(fa):
    run_fp8(fa, 1, 4, 1024, 1024, 128, True, 1410, exact_check=True)
    run_fp8(fa, 1, 4, 1024, 1024, 128, False, 1411, exact_check=True)
    run_fp8(fa, 1, 2, 1000, 1000, 128, False, 1412, q_sigma=8.0)
    run_fp8(fa, 1, 2, 700, 700, 64, True, 1413, transform=False)


def test_full_size_workload_sampled(fa):
    w = fa_inputs.WORKLOADS["fp8_causal_b8h16_n4096_d128"]
    note("case " + w.name)
    q, k, v = fa_inputs.make_workload(w)
    signs = fa_inputs.make_signs(w.d, w.seed)
    pack = fa.fa_quantize_fp8(*to_dev(q, k, v), signs=signs.to(DEV))
    out, lse = fa.fa_fwd_fp8(pack, w.B, w.H, w.Nq, w.Nk, w.d, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rows = fa_inputs.sample_rows(w.B, w.H, w.Nq, 3000, seed=1420)
    ro, rl, _ = fp8.fp8_attention(q, k, v, w.scale, True, signs=signs.numpy(), rows=rows)
    o = out.reshape(-1, w.d).float().cpu().numpy()[rows].astype(np.float64)
    l = lse.reshape(-1).cpu().numpy()[rows].astype(np.float64)
    ro = ro.reshape(-1, w.d)[rows]
    rl = rl.reshape(-1)[rows]
    err, lerr = np.abs(o - ro), np.abs(l - rl)
    note("%s: max|dO|=%.3e mean|dO|=%.3e max|dLSE|=%.3e" % (w.name, err.max(), err.mean(), lerr.max()))
    assert err.max() <= FP8_MAX and err.mean() <= FP8_MEAN and lerr.max() <= FP8_LSE


def test_deterministic(fa):
    q, k, v = fa_inputs.make_qkv(1, 2, 500, 500, 128, "bf16", 1430)
    qd, kd, vd = to_dev(q, k, v)
    s = signs_dev(128, 1430)
    p1 = fa.fa_quantize_fp8(qd, kd, vd, signs=s)
    p2 = fa.fa_quantize_fp8(qd, kd, vd, signs=s)
    o1 = fa.fa_fwd_fp8(p1, 1, 2, 500, 500, 128, causal=True)
    o2 = fa.fa_fwd_fp8(p2, 1, 2, 500, 500, 128, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(o1[0], o2[0]) and torch.equal(o1[1], o2[1])
