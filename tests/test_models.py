"""The parity bars of the GPU tests, recomputed from committed CPU models of
the kernels' rounding points (tests/rounding_models.py) against the fp64
oracle.

* Backward ("9.4 FlashAttention 与 FlashMLA" section 9.4.5; the pages give
  no tolerance): on the shapes and seeds the GPU backward tests run, the
  model's per-gradient figures must lie within parity_util.BWD_TOL.
* FP8 forward (section 9.4.4; no tolerance either): on the shapes and seeds
  the GPU FP8 tests run, the model's max and mean |dO| against exact
  attention on the dequantised inputs must lie within FP8_MAX / FP8_MEAN,
  and its mean |dO| against exact attention on the original inputs within
  FP8_EXACT_MEAN.
* Long non-causal bf16 prefill with scores of spread 64 (the workload B1
  H32 N16384 d128, q ~ N(0, 8^2)): the margin of the 16-bit forward to its
  stated bar (max |dO| <= 2e-2) over four seeds, on the waves of 32 queries
  whose outputs are largest (where the bf16 rounding of O is coarsest) plus
  waves spread over the sequence.  Besides the model's error, each element
  gets the worst case of the final rounding: its error before the rounding
  plus half a bf16 unit at |O|.  That worst case must stay below the bar,
  so the margin does not rest on how the roundings happen to fall.

The figures are printed so that a run shows them.
"""
import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from oracle import fp8
import rounding_models as rm
from parity_util import BWD_TOL, FP8_EXACT_MEAN, FP8_LSE, FP8_MAX, FP8_MEAN, LSE_TOL, TOL

BWD_SHAPES = [(1, 2, 300, 300), (2, 1, 517, 200), (1, 1, 129, 300), (1, 3, 64, 64), (1, 1, 1, 77), (1, 2, 255, 1)]


def bwd_case(B, H, Nq, Nk, d, dtype, causal, seed, q_sigma=1.0, heads=None):
    """The model's (element, mean) figures per gradient tensor, compared as
    the GPU test compares (rms over the whole tensor; an all-zero reference
    gradient is skipped, the GPU test checks it by absolute error)."""
    q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, dtype, seed, q_sigma)
    g = fa_inputs.make_dout(B, H, Nq, d, dtype, seed)
    scale = fa_inputs.default_scale(d)
    bh = list(range(B * H)) if heads is None else list(heads)
    o, lse = oracle.attention(q, k, v, scale, causal)
    ref = oracle.attention_bwd(q, k, v, g, scale, causal, heads=np.array(bh) if heads is not None else None)
    flat = lambda t: t.reshape((B * H,) + tuple(t.shape[2:]))
    qf, kf, vf, gf = (flat(t.float()) for t in (q, k, v, g))
    of, lf = flat(torch.from_numpy(o)), flat(torch.from_numpy(lse))
    got = [[], [], []]
    for i in bh:
        ob = of[i].to(rm.TYPES[dtype]).float()
        for j, x in enumerate(rm.backward_model(qf[i], kf[i], vf[i], ob, lf[i].float(), gf[i], scale, causal, dtype)):
            got[j].append(x)
    out = []
    for j, r in enumerate(ref):
        r = np.asarray(r).reshape((len(bh),) + np.asarray(r).shape[-2:])
        if not np.any(r):
            continue
        out.append(rm.grad_errors(np.stack(got[j]), r))
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_backward_bar_covers_the_model(dtype):
    figures = []
    for d in (32, 64, 128):
        for causal in (False, True):
            for i, (B, H, Nq, Nk) in enumerate(BWD_SHAPES):
                figures += bwd_case(B, H, Nq, Nk, d, dtype, causal, 700 + i)
    if dtype == "bf16":
        for causal in (False, True):
            figures += bwd_case(1, 4, 1024, 1024, 128, "bf16", causal, 710)
        figures += bwd_case(1, 2, 1000, 1000, 128, "bf16", False, 711, q_sigma=8.0)
        # two heads of the full-size backward workload (B8 H16 N4096, causal)
        w = fa_inputs.WORKLOADS["bwd_causal_bf16_b8h16_n4096_d128"]
        q, k, v = fa_inputs.make_workload(w)
        figures += bwd_case_from(w, q, k, v, heads=[0, 77])
    elem = max(f[0] for f in figures)
    mean = max(f[1] for f in figures)
    print("backward %s model: max element error %.4f, max mean/rms %.2e; bar %s" % (dtype, elem, mean, BWD_TOL[dtype]))
    assert elem <= BWD_TOL[dtype][0] and mean <= BWD_TOL[dtype][1]


def bwd_case_from(w, q, k, v, heads):
    g = fa_inputs.make_dout(w.B, w.H, w.Nq, w.d, w.dtype, w.seed)
    out = []
    for i in heads:
        b, h = divmod(i, w.H)
        sl = lambda t: t[b:b + 1, h:h + 1].contiguous()
        qq, kk, vv, gg = sl(q), sl(k), sl(v), sl(g)
        o, lse = oracle.attention(qq, kk, vv, w.scale, w.causal)
        ref = oracle.attention_bwd(qq, kk, vv, gg, w.scale, w.causal)
        ob = torch.from_numpy(o[0, 0]).to(rm.TYPES[w.dtype]).float()
        mod = rm.backward_model(qq[0, 0].float(), kk[0, 0].float(), vv[0, 0].float(), ob,
                                torch.from_numpy(lse[0, 0]).float(), gg[0, 0].float(), w.scale, w.causal, w.dtype)
        out += [rm.grad_errors(x, np.asarray(r)[0, 0]) for x, r in zip(mod, ref)]
    return out


def fp8_case(q, k, v, scale, causal, signs, exact=False):
    """(max |dO|, mean |dO|, max |dLSE|, mean |dO| vs exact on the original
    inputs or None) of the FP8 model on [B, H, N, d] inputs."""
    ro, rl, qu = fp8.fp8_attention(q, k, v, scale, causal, signs=signs)
    B, H, Nq = qu["q8"].shape[:3]
    o_all = np.empty_like(ro)
    lerr = 0.0
    for b in range(B):
        for h in range(H):
            val = lambda c: torch.from_numpy(fp8.e4m3_values(c[b, h])).float()
            c = np.float32(np.float32(np.float32(scale * rm.LOG2E) * qu["dq"][b, h]) * qu["dk"][b, h])
            o, _, l = rm.forward_model(val(qu["q8"]), val(qu["k8"]), val(qu["v8"]), scale, causal,
                                       list(range((Nq + 31) // 32)), p_type=torch.float8_e4m3fn, bc=64,
                                       bound=256.0, c=c, out_type=torch.bfloat16, out_scale=float(qu["dv"][b, h]))
            o_all[b, h] = o
            lerr = max(lerr, float(np.abs(l - rl[b, h]).max()))
    err = np.abs(o_all - ro)
    ex = None
    if exact:
        eo, _ = oracle.attention(q, k, v, scale, causal)
        ex = float(np.abs(o_all - eo).mean())
    return float(err.max()), float(err.mean()), lerr, ex


def test_fp8_bar_covers_the_model():
    rows = []
    for d in (64, 128):
        for causal in (False, True):
            for B, H, Nq, Nk, seed in ((1, 2, 300, 517, 1400 + d), (2, 1, 129, 64, 1401 + d), (1, 1, 1, 77, 1402 + d)):
                q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, "bf16", seed)
                rows.append(fp8_case(q, k, v, fa_inputs.default_scale(d), causal,
                                     fa_inputs.make_signs(d, seed).numpy()))
    for causal, seed in ((True, 1410), (False, 1411)):
        q, k, v = fa_inputs.make_qkv(1, 4, 1024, 1024, 128, "bf16", seed)
        rows.append(fp8_case(q, k, v, fa_inputs.default_scale(128), causal, fa_inputs.make_signs(128, seed).numpy(),
                             exact=True))
    q, k, v = fa_inputs.make_qkv(1, 2, 1000, 1000, 128, "bf16", 1412, 8.0)
    rows.append(fp8_case(q, k, v, fa_inputs.default_scale(128), False, fa_inputs.make_signs(128, 1412).numpy()))
    q, k, v = fa_inputs.make_qkv(1, 2, 700, 700, 64, "bf16", 1413)
    rows.append(fp8_case(q, k, v, fa_inputs.default_scale(64), True, None))
    mx, mean, lse = max(r[0] for r in rows), max(r[1] for r in rows), max(r[2] for r in rows)
    ex = max(r[3] for r in rows if r[3] is not None)
    print("FP8 model: max|dO| %.4f, mean|dO| %.2e, max|dLSE| %.2e, mean|dO| vs exact %.2e; bars %g %g %g %g"
          % (mx, mean, lse, ex, FP8_MAX, FP8_MEAN, FP8_LSE, FP8_EXACT_MEAN))
    assert mx <= FP8_MAX and mean <= FP8_MEAN and lse <= FP8_LSE and ex <= FP8_EXACT_MEAN


@pytest.mark.parametrize("seed", [1004, 2004, 3004, 4004])
def test_long_prefill_margin_over_seeds(seed):
    N, d = 16384, 128
    scale = fa_inputs.default_scale(d)
    q, k, v = fa_inputs.make_qkv(1, 1, N, N, d, "bf16", seed, q_sigma=8.0)
    qf, kf, vf = q[0, 0].float(), k[0, 0].float(), v[0, 0].float()
    # the waves whose outputs are largest, from a float32 softmax of every row
    omax = torch.empty(N)
    for r0 in range(0, N, 2048):
        p = torch.softmax((qf[r0:r0 + 2048] @ kf.T) * scale, dim=-1)
        omax[r0:r0 + 2048] = (p @ vf).abs().max(-1).values
    risky = torch.argsort(omax.reshape(-1, 32).max(-1).values, descending=True)[:24].tolist()
    waves = sorted(set(risky + list(range(0, N // 32, N // 256))))
    rows = np.array([32 * w + i for w in waves for i in range(32)])
    ro, rl = oracle.attention(q, k, v, scale, False, rows=rows)
    # the 16-bit prefill kernel at d = 128: 32-key tiles, bf16 lazy bound 2^30
    o, o_pre, l = rm.forward_model(qf, kf, vf, scale, False, waves, p_type=torch.bfloat16, bc=32, bound=2.0 ** 30)
    err, pre = np.abs(o - ro), np.abs(o_pre - ro)
    a = np.abs(o_pre)
    half_unit = np.where(a > 0, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-30))) - 8), 0.0)
    worst = pre + half_unit
    max_tol, mean_tol = TOL["bf16"]
    print("seed %d, %d waves, max |O| %.2f: model max|dO| %.4f mean %.2e max|dLSE| %.2e; before the output "
          "rounding %.4f; worst-case rounding %.4f (bar %g)"
          % (seed, len(waves), np.abs(ro).max(), err.max(), err.mean(), np.abs(l - rl).max(), pre.max(),
             worst.max(), max_tol))
    assert err.max() <= max_tol and err.mean() <= mean_tol and np.abs(l - rl).max() <= LSE_TOL
    assert worst.max() <= max_tol
    # on the rows not modelled: every |V| < 8, so |O| < 8 (O is a convex
    # combination of value rows) and the output rounding adds at most 2^-6
    assert float(vf.abs().max()) < 8.0


def test_running_sum_bound_keeps_large_values_finite():
    """The bf16 lazy rescale bounds the lane's running sum of P since the
    last exact step, not each tile's sum: with scores that rise slowly along
    16384 keys (P up to 2^26 against the held max for most of the range)
    and positive values near 2^94, tile sums under 2^30 add up past the
    float32 range of the accumulator, while the running bound keeps it
    within 2^31 max|V|.  Exact attention is finite (about 1.05 * 2^94)."""
    N, d = 16384, 128
    scale = fa_inputs.default_scale(d)
    q, k, v = fa_inputs.make_rising_scores(N, d)
    ro, rl = oracle.attention(q, k, v, scale, False)
    q, k, v = (t[0, 0].float() for t in (q, k, v))
    assert np.isfinite(ro).all()
    o_tile, _, _ = rm.forward_model(q, k, v, scale, False, [0, 1], p_type=torch.bfloat16, bc=32,
                                    bound=2.0 ** 30, running=False)
    o_run, _, l_run = rm.forward_model(q, k, v, scale, False, [0, 1], p_type=torch.bfloat16, bc=32,
                                       bound=2.0 ** 30, running=True)
    assert not np.isfinite(o_tile).all()
    err = np.abs(o_run - ro[0, 0]) / 2.0 ** 94
    print("running bound: max |dO| / 2^94 = %.2e, max |dLSE| = %.2e" % (err.max(), np.abs(l_run - rl[0, 0]).max()))
    assert err.max() <= TOL["bf16"][0] and np.abs(l_run - rl[0, 0]).max() <= LSE_TOL

