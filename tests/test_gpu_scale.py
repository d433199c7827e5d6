"""GPU parity at negative and zero softmax scales, through the C ABI.

The caller passes the scale ("08. Triton Flash Attention": the kernel takes
sm_scale as an argument), so every entry point accepts any finite scale.
The kernels take the row max before scaling and therefore fold the sign of
the scale into the operand they hold in registers (Q, or K in the dK/dV
kernel); a zero scale zeroes that operand.  Each path is compared with the
fp64 oracle at the same tolerances as at the default scale, and the fold is
checked to be exact: a negative scale gives the same bits as the positive
scale applied to -q.
"""
import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from oracle import fp8
from parity_util import DEV, FP8_LSE, FP8_MAX, FP8_MEAN, LSE_TOL, compare, note, to_dev
from test_gpu_backward import compare_grad
from test_gpu_paged import run_paged

pytestmark = pytest.mark.gpu

SCALES = [-0.125, 0.0, -1.0]


@pytest.fixture(scope="module")
def fa():
    import io_aware_amd
    return io_aware_amd


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("bf16", 32), ("f32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill(fa, scale, dtype, d, causal):
    if dtype == "f32" and abs(scale) > 0.125:
        # scores of spread 16 (LSE near 60) put float32 exp2 and log past the
        # 1e-5 bar whatever the sign; the fold itself is checked bit for bit below
        pytest.skip("the float32 bar holds for scores of unit spread")
    for i, (B, H, Nq, Nk) in enumerate([(1, 2, 300, 517), (2, 1, 517, 300), (1, 1, 1, 77)]):
        if Nq == 1 and not causal and dtype != "f32":
            continue  # the decode shape is covered below
        label = "scale %g %s d%d causal=%d B%d H%d Nq%d Nk%d" % (scale, dtype, d, causal, B, H, Nq, Nk)
        note("case " + label)
        q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, dtype, 2100 + i, q_sigma=1.0 if dtype == "f32" else 2.0)
        out, lse = fa.fa_fwd(*to_dev(q, k, v), scale=scale, causal=causal)
        torch.cuda.synchronize()
        compare(out, lse, *oracle.attention(q, k, v, scale, causal), dtype, label)


@pytest.mark.parametrize("scale", SCALES)
def test_split_prefill(fa, scale, monkeypatch):
    # a grid of 2 workgroups over 8192 keys: the key range is split
    monkeypatch.setenv("FA_PREFILL_SPLIT", "7")
    q, k, v = fa_inputs.make_qkv(1, 2, 100, 3000, 128, "bf16", 2110)
    label = "split prefill scale %g" % scale
    note("case " + label)
    out, lse = fa.fa_fwd(*to_dev(q, k, v), scale=scale, causal=False)
    torch.cuda.synchronize()
    compare(out, lse, *oracle.attention(q, k, v, scale, False), "bf16", label)


@pytest.mark.parametrize("scale", SCALES)
def test_decode(fa, scale):
    q, k, v = fa_inputs.make_qkv(4, 8, 1, 3000, 128, "bf16", 2120, q_sigma=3.0)
    label = "decode scale %g" % scale
    note("case " + label)
    qd, kd, vd = to_dev(q, k, v)
    out, lse = fa.fa_fwd(qd, kd, vd, scale=scale)
    out2, lse2 = fa.fa_fwd_splitkv(qd, kd, vd, 5, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention(q, k, v, scale, False)
    compare(out, lse, *ref, "bf16", label)
    compare(out2, lse2, *ref, "bf16", label + " (5 chunks)")


@pytest.mark.parametrize("scale", SCALES)
def test_paged_decode(fa, scale):
    w = fa_inputs.PAGED_WORKLOADS["paged_mixed_f16_b6h4_len1000_d64_bs16_split8"]
    q, kc, vc, table, lens = fa_inputs.make_paged(w)
    run_paged(fa, q, kc, vc, table, lens, w.num_splits, scale, w.dtype, "paged scale %g" % scale)


@pytest.mark.parametrize("scale", SCALES)
def test_varlen(fa, scale):
    w = fa_inputs.VARLEN_WORKLOADS["varlen_mixed_f16_s9h4_len0to700_d64"]
    label = "varlen scale %g" % scale
    note("case " + label)
    q, k, v, cq, ck = fa_inputs.make_varlen(w)
    out, lse = fa.fa_fwd_varlen(*to_dev(q, k, v, cq, ck), scale=scale, causal=w.causal)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.varlen_attention(q, k, v, cq, ck, scale, w.causal)
    empty = np.isneginf(ref_l[0])
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    assert (o[empty] == 0).all() and np.isneginf(l[:, empty]).all()
    keep = ~empty
    compare(torch.from_numpy(o[keep]), torch.from_numpy(np.ascontiguousarray(l[:, keep])), ref_o[keep],
            ref_l[:, keep], w.dtype, label)


@pytest.mark.parametrize("scale", [-0.088, 0.0])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8(fa, scale, causal):
    B, H, Nq, Nk, d = 1, 2, 300, 517, 128
    label = "fp8 scale %g causal=%d" % (scale, causal)
    note("case " + label)
    q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, "bf16", 2130)
    signs = fa_inputs.make_signs(d, 2130)
    pack = fa.fa_quantize_fp8(*to_dev(q, k, v), signs=signs.to(DEV))
    out, lse = fa.fa_fwd_fp8(pack, B, H, Nq, Nk, d, scale=scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl, _ = fp8.fp8_attention(q, k, v, scale, causal, signs=signs.numpy())
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    err, lerr = np.abs(o - ro), np.abs(l - rl)
    note("%s: max|dO|=%.3e mean|dO|=%.3e max|dLSE|=%.3e" % (label, err.max(), err.mean(), lerr.max()))
    assert np.isfinite(o).all() and np.isfinite(l).all()
    assert err.max() <= FP8_MAX and err.mean() <= FP8_MEAN and lerr.max() <= FP8_LSE, label


@pytest.mark.parametrize("scale", [-0.125, 0.0])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward(fa, scale, dtype, d, causal):
    B, H, Nq, Nk = 1, 2, 300, 277
    label = "bwd scale %g %s d%d causal=%d" % (scale, dtype, d, causal)
    note("case " + label)
    q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, dtype, 2140)
    g = fa_inputs.make_dout(B, H, Nq, d, dtype, 2140)
    qd, kd, vd, gd = to_dev(q, k, v, g)
    out, lse = fa.fa_fwd(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, out, gd, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(q, k, v, g, scale, causal)
    for name, x, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        compare_grad(x, r, dtype, "%s %s" % (label, name))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("f32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale_is_the_positive_scale_on_negated_q(fa, dtype, d, causal):
    # negation is exact and the products and nearest-even sums are odd
    # functions, so folding the sign into Q changes no bit
    q, k, v = fa_inputs.make_qkv(2, 2, 333, 400, d, dtype, 2150)
    qd, kd, vd = to_dev(q, k, v)
    o1, l1 = fa.fa_fwd(qd, kd, vd, scale=-0.2, causal=causal)
    o2, l2 = fa.fa_fwd((-qd).contiguous(), kd, vd, scale=0.2, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_zero_scale_gives_the_mean_of_visible_values(fa):
    q, k, v = fa_inputs.make_qkv(1, 2, 200, 200, 128, "bf16", 2160, q_sigma=8.0)
    out, lse = fa.fa_fwd(*to_dev(q, k, v), scale=0.0, causal=True)
    torch.cuda.synchronize()
    n = torch.arange(1, 201, dtype=torch.float64)
    mean = torch.cumsum(v.double(), dim=2) / n[None, None, :, None]
    assert (out.double().cpu() - mean).abs().max().item() <= 2e-2
    assert (lse.double().cpu() - torch.log(n)[None, None, :]).abs().max().item() <= LSE_TOL
