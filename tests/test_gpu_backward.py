"""GPU parity of the backward (``fa_bwd``) against the fp64 oracle
(``oracle.attention_bwd``), through the C ABI.

The forward runs on the GPU first (``fa_fwd``), as a caller would run it, and
its ``out`` and ``lse`` feed the backward; the oracle computes the exact
gradients from the same q, k, v and dO.

Tolerance.  The pages state none for gradients.  The bar comes from the
arithmetic the kernels do: P and dS are rounded to the 16-bit type before
their products, accumulation is float32, D is formed from the stored (16-bit)
O, and outputs are rounded to nearest even.  tests/rounding_models.py models
exactly those rounding points on the CPU; on the cases below (the same
shapes and seeds) it gives, per gradient tensor, an element error
|x - x_ref| / (|x_ref| + rms(x_ref)) of at most 0.070 in bf16 and 0.0065 in
fp16, and a mean error of at most 2.8e-3 * rms(x_ref) in bf16 and 3.4e-4 *
rms(x_ref) in fp16 (tests/test_models.py recomputes them).  The tests allow
about twice those figures (parity_util.BWD_TOL):

    max |x - x_ref| / (|x_ref| + rms)  <=  0.125 (bf16), 0.016 (fp16)
    mean |x - x_ref|                   <=  6e-3 * rms (bf16), 1e-3 * rms (fp16)
"""
import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from parity_util import DEV, compare_grad, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import io_aware_amd
    return io_aware_amd


def run_bwd(fa, B, H, Nq, Nk, d, dtype, causal, seed, q_sigma=1.0, label=None):
    label = label or "bwd B%d H%d Nq%d Nk%d d%d %s causal=%d" % (B, H, Nq, Nk, d, dtype, causal)
    note("case " + label)
    q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, dtype, seed, q_sigma)
    g = fa_inputs.make_dout(B, H, Nq, d, dtype, seed)
    scale = fa_inputs.default_scale(d)
    qd, kd, vd, gd = to_dev(q, k, v, g)
    out, lse = fa.fa_fwd(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, out, gd, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(q, k, v, g, scale, causal)
    for name, x, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        compare_grad(x, r, dtype, "%s %s" % (label, name))
    return (q, k, v, g), (dq, dk, dv), ref


SHAPES = [(1, 2, 300, 300), (2, 1, 517, 200), (1, 1, 129, 300), (1, 3, 64, 64), (1, 1, 1, 77), (1, 2, 255, 1)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_shapes(fa, dtype, d, causal):
    for i, (B, H, Nq, Nk) in enumerate(SHAPES):
        run_bwd(fa, B, H, Nq, Nk, d, dtype, causal, seed=700 + i)


@pytest.mark.parametrize("causal", [False, True])
def test_medium_bf16(fa, causal):
    run_bwd(fa, 1, 4, 1024, 1024, 128, "bf16", causal, seed=710)


def test_large_scores_bf16(fa):
    run_bwd(fa, 1, 2, 1000, 1000, 128, "bf16", False, seed=711, q_sigma=8.0)


def test_keys_no_query_sees_get_zero(fa):
    # causal with Nk > Nq: keys >= Nq are after every query
    (q, k, v, g), (dq, dk, dv), _ = run_bwd(fa, 1, 2, 100, 300, 64, "bf16", True, seed=712)
    assert (dk[:, :, 100:] == 0).all() and (dv[:, :, 100:] == 0).all()


def test_full_size_workload_sampled_heads(fa):
    w = fa_inputs.WORKLOADS["bwd_causal_bf16_b8h16_n4096_d128"]
    note("case " + w.name)
    q, k, v = fa_inputs.make_workload(w)
    g = fa_inputs.make_dout(w.B, w.H, w.Nq, w.d, w.dtype, w.seed)
    qd, kd, vd, gd = to_dev(q, k, v, g)
    out, lse = fa.fa_fwd(qd, kd, vd, scale=w.scale, causal=True)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, out, gd, lse, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    # 16 of the 128 heads, two of each residue mod 8 (the workgroup order
    # gives each XCD its own heads), and 170 rows: tile and block edges plus
    # 160 drawn at random
    heads = np.arange(0, 128, 8) + np.arange(16) % 8
    rows = np.unique(np.r_[0, 1, 31, 32, 127, 128, 2047, 2048, 4094, 4095,
                           np.random.default_rng(5).integers(0, 4096, 160)])
    ref = oracle.attention_bwd(q, k, v, g, w.scale, True, heads=heads, q_idx=rows, k_idx=rows)
    hs, rs = torch.from_numpy(heads), torch.from_numpy(rows)
    for name, x, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        sel = x.reshape(w.B * w.H, w.Nq, w.d).cpu()[hs][:, rs]
        compare_grad(sel, r, w.dtype, "%s %s" % (w.name, name))


@pytest.mark.parametrize("variant", ["0", "1"])
@pytest.mark.parametrize("causal", [False, True])
def test_every_dkdv_variant(fa, variant, causal, monkeypatch):
    monkeypatch.setenv("FA_BWD_DKDV", variant)
    for d, dtype in ((128, "bf16"), (64, "f16"), (32, "bf16")):
        run_bwd(fa, 1, 2, 333, 300, d, dtype, causal, seed=740 + d,
                label="bwd variant %s d%d %s causal=%d" % (variant, d, dtype, causal))


def test_bitwise_deterministic(fa):
    q, k, v = fa_inputs.make_qkv(2, 2, 700, 700, 128, "bf16", 720)
    g = fa_inputs.make_dout(2, 2, 700, 128, "bf16", 720)
    qd, kd, vd, gd = to_dev(q, k, v, g)
    out, lse = fa.fa_fwd(qd, kd, vd, causal=True)
    a = fa.fa_bwd(qd, kd, vd, out, gd, lse, causal=True)
    b = fa.fa_bwd(qd, kd, vd, out, gd, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_guard_bands_untouched(fa):
    B, H, Nq, Nk, d = 1, 2, 333, 250, 64
    q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, "f16", 730)
    g = fa_inputs.make_dout(B, H, Nq, d, "f16", 730)
    qd, kd, vd, gd = to_dev(q, k, v, g)
    out, lse = fa.fa_fwd(qd, kd, vd, causal=False)
    pad = 4096
    bufs, views = [], []
    for n, shape in ((B * H * Nq * d, (B, H, Nq, d)), (B * H * Nk * d, (B, H, Nk, d)), (B * H * Nk * d, (B, H, Nk, d))):
        buf = torch.full((n + 2 * pad,), 7.0, dtype=torch.float16, device=DEV)
        bufs.append((buf, n))
        views.append(buf[pad:pad + n].view(*shape))
    fa.fa_bwd(qd, kd, vd, out, gd, lse, causal=False, dq=views[0], dk=views[1], dv=views[2])
    torch.cuda.synchronize()
    for buf, n in bufs:
        assert (buf[:pad].float() == 7.0).all() and (buf[pad + n:].float() == 7.0).all()
    ref = oracle.attention_bwd(q, k, v, g, fa_inputs.default_scale(d), False)
    for name, x, r in zip(("dQ", "dK", "dV"), views, ref):
        compare_grad(x, r, "f16", "guard bands " + name)
