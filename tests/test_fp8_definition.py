"""The FP8 quantiser of the oracle (``oracle.fp8``) against the plain
definition, computed in fp64 and rounded once.

"9.4 FlashAttention 与 FlashMLA" section 9.4.4 (FP8 attention with
incoherent processing) and the readings of ``include/fa.h``:

    y    = x diag(s) H_d / sqrt(d)        (Q and K; V is not transformed)
    amax = max |y| over one (batch, head)
    code = RNE_E4M3(clamp(y * 448 / amax, -448, 448))

Here H_d is built from its recursive definition as an explicit matrix, y is
one fp64 matrix product, amax and the scaling are fp64, and the E4M3
rounding is applied once to the fp64 value, against the table of E4M3 values
built from the format's definition (sign, 4-bit exponent with bias 7, 3-bit
mantissa, subnormals, 448 the largest finite value), with ties to the even
code.  Nothing here calls the oracle's transform or torch's float8 cast.

The oracle takes its decisions in float32 (the butterfly stage by stage, one
multiply by fp32(1/sqrt d), one division 448/amax, one multiply), the same
order as the library's kernel.  Its code may differ from the definition's
only where the fp64 value lies so close to a midpoint between two E4M3
values that the float32 error can carry it across.  The bound used per
element is a running error bound of the float32 butterfly (each stage's
a +- b adds its own rounding, u |a +- b| with u = 2^-24, to the bounds of a
and b), plus one rounding each for the 1/sqrt(d) multiply, the scale and
the scaling multiply, plus the observed shift of the float32 amax.  Every
mismatch must be a pair of neighbouring codes whose midpoint lies within
that bound of the fp64 value; the counts are printed.
"""
import math

import numpy as np
import pytest

import fa_inputs
from oracle import fp8

U = 2.0 ** -24  # unit roundoff of float32


def e4m3_table():
    """(code, value) of every finite E4M3 code, from the format definition."""
    codes, vals = [], []
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 0x7
        if e == 0xF and m == 0x7:
            continue  # NaN
        mag = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        codes.append(c)
        vals.append(sign * mag)
    return np.array(codes), np.array(vals)


def rne_e4m3(y):
    """fp64 values (|y| <= 448) -> E4M3 values, nearest with ties to the
    even code, from the table (one rounding of the fp64 value)."""
    codes, vals = e4m3_table()
    keep = vals >= 0
    pos_v, pos_c = vals[keep], codes[keep]
    order = np.argsort(pos_v)
    pos_v, pos_c = pos_v[order], pos_c[order]
    pos_v, first = np.unique(pos_v, return_index=True)
    pos_c = pos_c[first]
    a = np.abs(y)
    assert (a <= 448.0).all()
    hi = np.clip(np.searchsorted(pos_v, a, side="left"), 1, len(pos_v) - 1)
    lo = hi - 1
    dlo, dhi = a - pos_v[lo], pos_v[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (pos_c[hi] % 2 == 0))
    mag = np.where(pick_hi, pos_v[hi], pos_v[lo])
    return np.sign(y) * mag


def hadamard(d):
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def butterfly_error_bound(x):
    """Per-element bound on |fl32 butterfly(x) - exact| / u: the running
    bound A of each stage output a +- b is A(a) + A(b) + |a +- b|."""
    y = np.asarray(x, dtype=np.float64).copy()
    a = np.zeros_like(y)
    d = y.shape[-1]
    h = 1
    while h < d:
        ys = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        As = a.reshape(ys.shape)
        s0, s1 = ys[..., 0, :] + ys[..., 1, :], ys[..., 0, :] - ys[..., 1, :]
        a0 = As[..., 0, :] + As[..., 1, :]
        ys = np.stack([s0, s1], axis=-2)
        As = np.stack([a0 + np.abs(s0), a0 + np.abs(s1)], axis=-2)
        y = ys.reshape(y.shape)
        a = As.reshape(y.shape)
        h *= 2
    return a


def check_head(x, signs, label):
    """x [N, d] (float32 values of one head), signs [d] or None.  Returns
    (mismatches, elements)."""
    x = np.asarray(x, dtype=np.float32)
    N, d = x.shape
    xs = x.astype(np.float64) * (1.0 if signs is None else np.asarray(signs, dtype=np.float64))
    if signs is None:
        y64 = xs
        bound_t = np.zeros_like(y64)  # no transform: the float32 values are exact
    else:
        y64 = xs @ hadamard(d) / math.sqrt(d)
        # butterfly rounding, then the multiply by fp32(1/sqrt d): its own
        # rounding and the rounding of the constant
        bound_t = U * butterfly_error_bound(xs) / math.sqrt(d) + 2 * U * np.abs(y64)
    amax64 = np.abs(y64).max()
    # the oracle (float32 decisions) on this head alone
    codes, desc = fp8.quantize_heads((fp8.incoherent_transform(x, signs) if signs is not None else x)[None, None])
    codes, desc = codes[0, 0], float(desc[0, 0])
    amax32 = float(np.abs(fp8.incoherent_transform(x, signs) if signs is not None else x).max())
    # descale: fp32(amax32 / 448), amax32 within the bound of amax64
    assert abs(amax32 - amax64) <= bound_t.max() + 1e-300, label
    assert abs(desc * 448.0 - amax32) <= 2 * U * amax32, label
    ys64 = y64 * (448.0 / amax64)
    want = rne_e4m3(np.clip(ys64, -448.0, 448.0))
    got = fp8.e4m3_values(codes)
    bad = got != want
    # the float32 scaled value differs from ys64 by at most this much
    win = (448.0 / amax32) * (bound_t + 3 * U * np.abs(y64)) * (1 + 1e-6) + np.abs(ys64) * abs(amax64 / amax32 - 1)
    if bad.any():
        g, w, v, e = got[bad], want[bad], ys64[bad], win[bad]
        # neighbours: no E4M3 value strictly between the two
        _, table = e4m3_table()
        lo, hi = np.minimum(g, w), np.maximum(g, w)
        between = ((table[None, :] > lo[:, None]) & (table[None, :] < hi[:, None])).any(axis=1)
        assert not between.any(), "%s: a code off by more than one step" % label
        mid = (g + w) / 2
        assert (np.abs(v - mid) <= e).all(), "%s: a mismatch outside the float32 error bound (%.3e > %.3e)" % (
            label, np.abs(v - mid).max(), e[np.argmax(np.abs(v - mid) - e)])
    return int(bad.sum()), x.size


@pytest.mark.parametrize("tensor", ["q", "k", "v"])
def test_codes_of_the_fp8_workload_equal_the_definition(tensor):
    # whole heads of the FP8 workload's seeded inputs (B8 H16 N4096 d128);
    # Q and K carry the transform, V does not
    w = fa_inputs.WORKLOADS["fp8_causal_b8h16_n4096_d128"]
    q, k, v = fa_inputs.make_workload(w)
    x = {"q": q, "k": k, "v": v}[tensor]
    signs = fa_inputs.make_signs(w.d, w.seed).numpy() if tensor != "v" else None
    bad = total = 0
    for b, h in [(0, 0), (3, 7), (7, 15)]:
        m, n = check_head(x[b, h].float().numpy(), signs, "%s head (%d, %d)" % (tensor, b, h))
        bad, total = bad + m, total + n
    print("%s: %d of %d codes differ from the fp64 definition, each inside the float32 bound" % (tensor, bad, total))
    assert bad <= total * 1e-4


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("sigma", [1.0, 8.0])
def test_codes_equal_the_definition_on_other_inputs(d, sigma):
    q, _, _ = fa_inputs.make_qkv(1, 2, 1000, 1, d, "bf16", 1500 + d, q_sigma=sigma)
    signs = fa_inputs.make_signs(d, 1500)
    for h in range(2):
        m, n = check_head(q[0, h].float().numpy(), signs.numpy(), "d%d sigma %g head %d" % (d, sigma, h))
        print("d%d sigma %g head %d: %d of %d codes differ, each inside the float32 bound" % (d, sigma, h, m, n))
        assert m <= n * 1e-4


def test_definition_detects_a_planted_mistake():
    # the sign flips applied after the Hadamard matrix instead of before are
    # another orthogonal transform: the codes differ far from any midpoint
    rng = np.random.default_rng(7)
    d = 64
    x = rng.standard_normal((200, d)).astype(np.float32)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0).astype(np.float32)
    y_wrong = (x.astype(np.float64) @ hadamard(d)) * s / math.sqrt(d)
    codes, _ = fp8.quantize_heads(fp8.incoherent_transform(x, s)[None, None])
    got = fp8.e4m3_values(codes[0, 0])
    want = rne_e4m3(np.clip(y_wrong * 448.0 / np.abs(y_wrong).max(), -448, 448))
    assert (got != want).mean() > 0.5


def test_rne_table_matches_the_format():
    codes, vals = e4m3_table()
    assert len(codes) == 254 and vals.max() == 448.0 and vals.min() == -448.0
    pos = np.unique(vals[vals > 0])
    assert pos[0] == 2.0 ** -9 and len(pos) == 126
    # ties go to the even code: 0.5 * (1 + 1.125) sits between codes 0x38 and 0x39
    assert rne_e4m3(np.array([1.0625]))[0] == 1.0
    assert rne_e4m3(np.array([1.1875]))[0] == 1.25   # between 1.125 (odd 0x39) and 1.25 (even 0x3A)
    assert rne_e4m3(np.array([-448.0, 440.0, 2.0 ** -10]))[0] == -448.0
    assert rne_e4m3(np.array([2.0 ** -10]))[0] == 0.0    # half the smallest subnormal: tie to even zero
