"""Shared helpers of the GPU parity tests: the tolerances and the
element-by-element comparison against the fp64 oracle.

Tolerances on O and LSE (absolute, after widening the GPU outputs to fp64):
float32 path max |dO| <= 1e-5; fp16 / bf16 paths max |dO| <= 2e-2 and
mean |dO| <= 2e-3; LSE max |dLSE| <= 1e-3 on every path.
"""
import sys

import numpy as np

TOL = {"f32": (1e-5, None), "f16": (2e-2, 2e-3), "bf16": (2e-2, 2e-3)}
LSE_TOL = 1e-3
DEV = "cuda:0"

# Bars with no stated tolerance on the pages, each about twice the largest
# figure of a CPU model of the kernels' rounding points on the cases the
# GPU tests run (tests/rounding_models.py; recomputed by tests/test_models.py,
# which asserts that every bar covers its model):
# * backward, per gradient tensor: (max |x - ref| / (|ref| + rms(ref)),
#   mean |x - ref| / rms(ref)) for bf16 and fp16;
# * FP8 forward against exact attention on the dequantised inputs: max and
#   mean |dO|, max |dLSE|; and mean |dO| against exact attention on the
#   original inputs (quantisation included).
BWD_TOL = {"bf16": (0.125, 6e-3), "f16": (0.016, 1e-3)}
FP8_MAX, FP8_MEAN, FP8_LSE = 0.12, 8e-3, 1e-3
FP8_EXACT_MEAN = 1e-2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def compare(out, lse, ref_o, ref_l, dtype, label):
    o = out.detach().float().cpu().numpy().astype(np.float64).reshape(ref_o.shape)
    l = lse.detach().float().cpu().numpy().astype(np.float64).reshape(ref_l.shape)
    assert np.isfinite(o).all(), label + ": non-finite O"
    assert np.isfinite(l).all(), label + ": non-finite LSE"
    err = np.abs(o - ref_o)
    lerr = np.abs(l - ref_l)
    max_tol, mean_tol = TOL[dtype]
    note("%s: max|dO|=%.3e mean|dO|=%.3e max|dLSE|=%.3e" % (label, err.max(), err.mean(), lerr.max()))
    assert err.max() <= max_tol, "%s: max|dO| %.3e > %.1e" % (label, err.max(), max_tol)
    if mean_tol is not None:
        assert err.mean() <= mean_tol, "%s: mean|dO| %.3e > %.1e" % (label, err.mean(), mean_tol)
    assert lerr.max() <= LSE_TOL, "%s: max|dLSE| %.3e > %.1e" % (label, lerr.max(), LSE_TOL)


def to_dev(*ts):
    return [t.to(DEV).contiguous() for t in ts]


def compare_grad(x, ref, dtype, label):
    """A gradient against the fp64 backward oracle: per element
    |d| / (|ref| + rms(ref)) and the mean |d| / rms(ref) within BWD_TOL."""
    x = x.detach().float().cpu().numpy().astype(np.float64).reshape(ref.shape)
    assert np.isfinite(x).all(), label + ": non-finite gradient"
    err = np.abs(x - ref)
    rms = float(np.sqrt((ref ** 2).mean()))
    if rms == 0.0:
        # an exactly-zero gradient (a single key: P = 1, dS = 0) comes out as
        # float32 rounding noise of dP - D, far below 16-bit resolution
        assert err.max() <= 1e-4, "%s: %.3e where the gradient is 0" % (label, err.max())
        return
    elem = (err / (np.abs(ref) + rms)).max()
    max_tol, mean_tol = BWD_TOL[dtype]
    note("%s: rms=%.3e max|d|=%.3e elem=%.3e mean/rms=%.3e" % (label, rms, err.max(), elem, err.mean() / rms))
    assert elem <= max_tol, "%s: max |d|/(|ref|+rms) %.3e > %.3e" % (label, elem, max_tol)
    assert err.mean() <= mean_tol * rms, "%s: mean |d| %.3e > %.1e * rms" % (label, err.mean(), mean_tol)
