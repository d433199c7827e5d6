"""GPU parity beyond 2^31 elements per tensor: the dense forward, the
split-KV decode, the paged decode, the backward and the FP8 forward index
their tensors with 64-bit offsets.  The tensors here
hold more than 2^31 elements (4 GiB and more in bf16); heads past element 2^31
are compared with the fp64 oracle on sampled query rows (a head at a time:
the oracle sees that head's K and V in full).

Inputs are drawn on the GPU by fa_inputs.make_qkv_device (seeded); the
sampled heads are copied to the host for the oracle.
"""
import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from oracle import fp8
from parity_util import DEV, FP8_LSE, FP8_MAX, FP8_MEAN, compare, compare_grad, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import io_aware_amd
    return io_aware_amd


def _check_heads(q, k, v, out, lse, heads, rows, scale, causal, label):
    """The oracle on whole heads (their K and V in full), at the sampled rows."""
    H, d = q.shape[1], q.shape[3]
    for bh in heads:
        b, h = divmod(bh, H)
        ref_o, ref_l = oracle.attention(q[b, h].cpu()[None, None], k[b, h].cpu()[None, None],
                                        v[b, h].cpu()[None, None], scale, causal, rows=np.asarray(rows))
        compare(out[b, h, rows], lse[b, h, rows], ref_o.reshape(len(rows), d), ref_l.reshape(len(rows)), "bf16",
                "%s head %d" % (label, bh))


@pytest.mark.parametrize("causal", [False, True])
def test_dense_forward_past_2_31_elements(fa, causal):
    B, H, N, d = 2, 1025, 8192, 128          # 2*1025*8192*128 = 2^31 + 2^24 elements per tensor
    assert B * H * N * d > 2 ** 31
    note("case dense B%d H%d N%d d%d causal=%d (sampled heads past element 2^31)" % (B, H, N, d, causal))
    q, k, v = fa_inputs.make_qkv_device(B, H, N, N, d, "bf16", seed=4242, device=DEV)
    scale = fa_inputs.default_scale(d)
    out, lse = fa.fa_fwd(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    first_past = (2 ** 31) // (N * d)                      # first head starting at or past element 2^31
    heads = sorted({first_past, first_past + 1, B * H - 1})
    rows = [0, 1, 127, 128, 4095, 4096, 8190, 8191]
    _check_heads(q, k, v, out, lse, heads, rows, scale, causal, "dense")
    assert torch.isfinite(out[-1, -1].float()).all() and torch.isfinite(lse[-1, -1]).all()


def test_decode_past_2_31_elements(fa):
    B, H, Nk, d = 4, 1025, 8192, 128         # 4*1025*8192*128 = 2^32 + 2^25 elements per K and V
    assert B * H * Nk * d > 2 ** 31
    note("case decode B%d H%d Nk%d d%d (sampled heads past element 2^31)" % (B, H, Nk, d))
    q, k, v = fa_inputs.make_qkv_device(B, H, 1, Nk, d, "bf16", seed=4343, device=DEV)
    scale = fa_inputs.default_scale(d)
    out, lse = fa.fa_fwd_splitkv(q, k, v, 32, scale=scale)
    torch.cuda.synchronize()
    first_past = (2 ** 31) // (Nk * d)
    for bh in sorted({first_past, first_past + 1, B * H - 1}):
        b, h = divmod(bh, H)
        ref_o, ref_l = oracle.attention(q[b, h].cpu()[None, None], k[b, h].cpu()[None, None],
                                        v[b, h].cpu()[None, None], scale, False)
        compare(out[b, h], lse[b, h], ref_o.reshape(1, d), ref_l.reshape(1), "bf16", "decode head %d" % bh)


def test_backward_past_2_31_elements(fa):
    B, H, N, d = 33, 128, 4096, 128          # 33*128*4096*128 = 2^31 + 2^26 elements per tensor
    assert B * H * N * d > 2 ** 31
    note("case backward B%d H%d N%d d%d causal (sampled heads past element 2^31)" % (B, H, N, d))
    q, k, v = fa_inputs.make_qkv_device(B, H, N, N, d, "bf16", seed=4444, device=DEV)
    g = fa_inputs.make_qkv_device(B, H, N, 1, d, "bf16", seed=4445, device=DEV)[0]   # dO, Q-shaped
    scale = fa_inputs.default_scale(d)
    out, lse = fa.fa_fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv = fa.fa_bwd(q, k, v, out, g, lse, scale=scale, causal=True)
    torch.cuda.synchronize()
    first_past = (2 ** 31) // (N * d)
    rows = np.array([0, 1, 31, 32, 127, 128, 2047, 2048, 4094, 4095])
    for bh in sorted({first_past, first_past + 1, B * H - 1}):
        b, h = divmod(bh, H)
        one = [t[b, h].cpu()[None, None] for t in (q, k, v, g)]
        ref = oracle.attention_bwd(*one, scale, True, heads=np.array([0]), q_idx=rows, k_idx=rows)
        r = torch.from_numpy(rows)
        for name, x, rf in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            compare_grad(x[b, h].cpu()[r][None], rf, "bf16", "backward head %d %s" % (bh, name))


def test_fp8_past_2_31_elements(fa):
    B, H, N, d = 33, 128, 4096, 128          # every bf16 input 2^31 + 2^26 elements, every code array as many bytes
    assert B * H * N * d > 2 ** 31
    note("case fp8 B%d H%d N%d d%d causal (sampled heads past element 2^31)" % (B, H, N, d))
    q, k, v = fa_inputs.make_qkv_device(B, H, N, N, d, "bf16", seed=4646, device=DEV)
    signs = fa_inputs.make_signs(d, 4646)
    scale = fa_inputs.default_scale(d)
    pack = fa.fa_quantize_fp8(q, k, v, signs=signs.to(DEV))
    out, lse = fa.fa_fwd_fp8(pack, B, H, N, N, d, scale=scale, causal=True)
    torch.cuda.synchronize()
    first_past = (2 ** 31) // (N * d)
    rows = np.array([0, 1, 63, 64, 127, 128, 2047, 2048, 4094, 4095])
    for bh in sorted({first_past, first_past + 1, B * H - 1}):
        b, h = divmod(bh, H)
        one = [t[b, h].cpu()[None, None] for t in (q, k, v)]   # per-head scales: one head is self-contained
        ro, rl, _ = fp8.fp8_attention(*one, scale, True, signs=signs.numpy(), rows=rows)
        o = out[b, h].float().cpu().numpy()[rows].astype(np.float64)
        l = lse[b, h].cpu().numpy()[rows].astype(np.float64)
        err = np.abs(o - ro.reshape(-1, d)[rows])
        lerr = np.abs(l - rl.reshape(-1)[rows])
        note("fp8 head %d: max|dO|=%.3e mean|dO|=%.3e max|dLSE|=%.3e" % (bh, err.max(), err.mean(), lerr.max()))
        assert err.max() <= FP8_MAX and err.mean() <= FP8_MEAN and lerr.max() <= FP8_LSE, "fp8 head %d" % bh


def test_paged_decode_past_2_31_elements(fa):
    # caches [num_blocks, H, 16, 128] of 33280 blocks: 2^31 + 2^25 elements each;
    # block 32768 and above start at or past element 2^31
    H, bs, d, B, max_len = 32, 16, 128, 4, 8192
    per_block = H * bs * d
    num_blocks = 2 ** 31 // per_block + 512
    assert num_blocks * per_block > 2 ** 31
    note("case paged B%d H%d bs%d d%d num_blocks %d (sequence 0 in blocks past element 2^31)" % (B, H, bs, d, num_blocks))
    g = torch.Generator(device=DEV).manual_seed(4747)
    kc = torch.empty((num_blocks, H, bs, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    for t in (kc, vc):
        for i in range(0, num_blocks, 1024):
            t[i:i + 1024].copy_(torch.randn(t[i:i + 1024].shape, generator=g, device=DEV))
    q = torch.randn((B, H, 1, d), generator=g, device=DEV).to(torch.bfloat16)
    lens = torch.tensor([max_len, 8000, 5000, max_len], dtype=torch.int32)
    max_blocks = max_len // bs
    hg = torch.Generator().manual_seed(4747)
    first_past = 2 ** 31 // per_block
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    table[0] = first_past + torch.randperm(512, generator=hg)[:max_blocks].to(torch.int32)
    rest = torch.randperm(first_past, generator=hg)
    for b in range(1, B):
        nb = -(-int(lens[b]) // bs)
        table[b, :nb] = rest[(b - 1) * max_blocks:(b - 1) * max_blocks + nb].to(torch.int32)
    scale = fa_inputs.default_scale(d)
    out, lse = fa.fa_fwd_paged_decode(q, kc, vc, table.to(DEV), lens.to(DEV), 32, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    for b in (0, 2):
        # the oracle gets the sequence's blocks, copied to the host one by one,
        # and the table remapped onto them
        nb = -(-int(lens[b]) // bs)
        blocks = table[b, :nb].tolist()
        hk = torch.stack([kc[x].cpu() for x in blocks])
        hv = torch.stack([vc[x].cpu() for x in blocks])
        htab = torch.arange(nb, dtype=torch.int32)[None]
        ref_o, ref_l = oracle.paged_decode(q[b:b + 1].cpu(), hk, hv, htab, lens[b:b + 1], scale)
        compare(out[b, :, 0].float().cpu(), lse[b].cpu(), ref_o[0], ref_l[0], "bf16", "paged sequence %d" % b)
