"""The seeded input generator: deterministic, correctly shaped and rounded."""
import numpy as np
import torch

import fa_inputs


def test_same_seed_same_tensors():
    a = fa_inputs.make_qkv(1, 2, 33, 40, 16, "bf16", seed=5)
    b = fa_inputs.make_qkv(1, 2, 33, 40, 16, "bf16", seed=5)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    c = fa_inputs.make_qkv(1, 2, 33, 40, 16, "bf16", seed=6)
    assert not torch.equal(a[0], c[0])


def test_shapes_dtypes_and_rounding():
    q, k, v = fa_inputs.make_qkv(2, 3, 10, 20, 8, "f16", seed=1, q_sigma=8.0)
    assert q.shape == (2, 3, 10, 8) and k.shape == (2, 3, 20, 8) and v.shape == k.shape
    assert q.dtype == k.dtype == v.dtype == torch.float16
    # the values are the float32 draws rounded to nearest fp16 (ties to even)
    g = torch.Generator().manual_seed(1)
    q32 = torch.randn((2, 3, 10, 8), generator=g) * 8.0
    ref = q32.numpy().astype(np.float16)            # numpy's cast rounds to nearest even
    np.testing.assert_array_equal(q.numpy(), ref)


def test_scale_is_float32_inverse_sqrt():
    for d in (32, 64, 128):
        s = fa_inputs.default_scale(d)
        assert s == float(np.float32(1.0 / np.sqrt(d)))


def test_workloads_have_distinct_seeds_and_valid_sizes():
    seeds = [w.seed for w in fa_inputs.WORKLOADS.values()]
    assert len(set(seeds)) == len(seeds)
    for w in fa_inputs.WORKLOADS.values():
        assert w.d in (32, 64, 128) and w.dtype in fa_inputs.DTYPES


def test_sample_rows_cover_boundaries_and_stay_in_range():
    rows = fa_inputs.sample_rows(2, 8, 1000, 500, seed=3)
    assert rows.min() >= 0 and rows.max() < 2 * 8 * 1000
    assert len(np.unique(rows)) == len(rows) == 500
    assert {0, 999, 63, 64}.issubset(set(rows.tolist()))
    assert 2 * 8 * 1000 - 1 in set(rows.tolist())
