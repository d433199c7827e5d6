"""fa_fwd_noalloc -- the forward for callers that cannot allocate -- against
fa_fwd and the fp64 oracle, through the C ABI.

Its split workspace is the library's static scratch array, shared by every
call on the GPU and left holding the last call's contents, so each case runs
two calls in a row, the second on a smaller input, and checks both.  Where
the split workspace fits the array the chunk count is fa_fwd's and the
results must be equal bit for bit; a split prefill too large for it takes
fewer chunks and is held to the oracle tolerance (max |dO| <= 2e-2, mean
|dO| <= 2e-3, max |dLSE| <= 1e-3).
"""
import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from parity_util import DEV, compare, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import io_aware_amd
    return io_aware_amd


def noalloc(fa, qd, kd, vd, scale, causal):
    out = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=DEV)
    fa.fa_fwd_noalloc(qd, kd, vd, out, lse, scale=scale, causal=causal)
    return out, lse


def check_pair(fa, shapes, causal, dtype, seed, label):
    """Two noalloc calls in a row (the second smaller), each against fa_fwd
    (bit for bit) and the oracle."""
    for i, (B, H, Nq, Nk, d) in enumerate(shapes):
        tag = "%s call %d: B%d H%d Nq%d Nk%d d%d" % (label, i + 1, B, H, Nq, Nk, d)
        note("case " + tag)
        q, k, v = fa_inputs.make_qkv(B, H, Nq, Nk, d, dtype, seed + i)
        qd, kd, vd = to_dev(q, k, v)
        scale = fa_inputs.default_scale(d)
        o1, l1 = noalloc(fa, qd, kd, vd, scale, causal)
        o2, l2 = fa.fa_fwd(qd, kd, vd, scale=scale, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), tag + ": differs from fa_fwd"
        rows = fa_inputs.sample_rows(B, H, Nq, 400, seed=seed + i)
        ref_o, ref_l = oracle.attention(q, k, v, scale, causal, rows=rows)
        r = torch.from_numpy(rows).to(DEV)
        compare(o1.reshape(-1, d)[r], l1.reshape(-1)[r], ref_o, ref_l, dtype, tag)


def test_decode_full_size_then_smaller(fa):
    # the decode workload (32 chunks of 256 keys, 8.45 MB of scratch), then a
    # smaller decode whose 5 chunks leave most of the array as the first call left it
    w = fa_inputs.WORKLOADS["decode_bf16_b16h32_nk8192_d128_split32"]
    check_pair(fa, [(w.B, w.H, 1, w.Nk, w.d), (2, 3, 1, 1200, 64)], False, "bf16", 3100, "decode")


def test_split_prefill_then_smaller(fa):
    # grids of 2 to 20 workgroups over key ranges of 64 tiles or more: the
    # key range is split into chunks merged through the scratch (the last
    # case's 22 tiles are split over the waves of each workgroup instead)
    check_pair(fa, [(1, 2, 128, 8192, 128), (1, 3, 100, 5000, 64)], False, "bf16", 3110, "split prefill")
    check_pair(fa, [(1, 1, 2500, 4000, 128), (1, 1, 700, 700, 128)], True, "f16", 3120, "split causal")


def test_prefill_without_scratch_and_f32_split(fa):
    # a 16-bit grid that needs no split workspace; then float32 grids below
    # one workgroup per CU, whose key ranges are split into chunks merged
    # through the scratch (40 chunks of 4 blocks, then 3 of 1; causal: 8, then 4)
    check_pair(fa, [(2, 4, 1000, 1000, 128), (1, 2, 300, 517, 64)], True, "bf16", 3130, "prefill")
    check_pair(fa, [(1, 2, 300, 5000, 32), (1, 2, 100, 77, 32)], False, "f32", 3140, "f32")
    check_pair(fa, [(1, 1, 256, 256, 64), (1, 1, 70, 130, 128)], True, "f32", 3150, "f32 causal")


def test_split_too_large_for_the_scratch_takes_fewer_chunks(fa):
    # fa_fwd would cut each Q block's 65536 keys into 32 chunks: 33.8 MB of
    # workspace, over the 16 MiB array, so the noalloc call takes 15 chunks
    B, H, Nq, Nk, d = 1, 16, 128, 65536, 128
    assert fa.fa_splitkv_workspace_bytes(B, H, Nq, d, 32) > fa.FA_NOALLOC_SCRATCH_BYTES
    for i, shape in enumerate([(B, H, Nq, Nk, d), (1, 2, 64, 9000, 128)]):
        tag = "oversized split call %d: B%d H%d Nq%d Nk%d d%d" % ((i + 1,) + shape)
        note("case " + tag)
        q, k, v = fa_inputs.make_qkv(*shape, "bf16", 3150 + i)
        qd, kd, vd = to_dev(q, k, v)
        scale = fa_inputs.default_scale(shape[4])
        o1, l1 = noalloc(fa, qd, kd, vd, scale, False)
        torch.cuda.synchronize()
        assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
        rows = fa_inputs.sample_rows(shape[0], shape[1], shape[2], 300, seed=3150 + i)
        ref_o, ref_l = oracle.attention(q, k, v, scale, False, rows=rows)
        r = torch.from_numpy(rows).to(DEV)
        compare(o1.reshape(-1, shape[4])[r], l1.reshape(-1)[r], ref_o, ref_l, "bf16", tag)


def test_calls_leave_device_memory_unchanged(fa):
    # after first calls (which look the array up and load the kernels),
    # further calls of any size allocate nothing: the device's free memory
    # does not move
    q, k, v = fa_inputs.make_qkv(16, 32, 1, 8192, 128, "bf16", 3160)
    qd, kd, vd = to_dev(q, k, v)
    qs, ks, vs = to_dev(*fa_inputs.make_qkv(1, 4, 128, 8192, 128, "bf16", 3161))
    out, lse = torch.empty_like(qd), torch.empty(qd.shape[:3], dtype=torch.float32, device=DEV)
    out2, lse2 = torch.empty_like(qs), torch.empty(qs.shape[:3], dtype=torch.float32, device=DEV)
    fa.fa_fwd_noalloc(qd, kd, vd, out, lse)
    fa.fa_fwd_noalloc(qs, ks, vs, out2, lse2)   # every kernel of both paths launched once
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        fa.fa_fwd_noalloc(qs, ks, vs, out2, lse2)
        fa.fa_fwd_noalloc(qd, kd, vd, out, lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    note("free device memory before %d after %d" % (free0, free1))
    assert free1 == free0


def test_rejects_a_decode_too_large_for_the_scratch(fa):
    # 1024 x 64 heads at d = 128: one chunk per head needs 33.8 MB
    B, H, d = 1024, 64, 128
    q = torch.zeros((B, H, 1, d), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, H, 4, d), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd_noalloc(q, k, k, out)
    assert e.value.status == fa.FA_ERR_WORKSPACE
