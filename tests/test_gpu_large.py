"""GPU parity beyond 2^31 elements per tensor: the dense forward and the
split-KV decode index q, k, v and out with 64-bit offsets.  The tensors here
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
from parity_util import DEV, compare, note

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
