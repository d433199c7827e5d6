"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph).

Every kernel of the library is enqueued on the caller's stream and none of
them clears memory with a memset, so a forward can be captured once and
replayed.  The library-owned split workspace (decode, and prefill grids too
small for the GPU) is allocated by the first call on a stream, so an eager
call on the capture's side stream comes first; varlen takes a caller
workspace.  Each test replays its graph several times with new inputs copied
into the captured buffers, with eager library work and synchronisations in
between, and requires every replay to equal (bit for bit: the kernels are
deterministic) an eager call on the same inputs.
"""
import itertools

import pytest
import torch

import fa_inputs

pytestmark = pytest.mark.gpu

from parity_util import DEV  # noqa: E402


@pytest.fixture(scope="module")
def fa():
    import io_aware_amd
    return io_aware_amd


def _capture(fn):
    """Warm ``fn`` up on a side stream (allocates the library workspace of
    that stream), then capture it into a graph on that same stream."""
    side = torch.cuda.Stream()                       # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):           # the stream whose workspace exists
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(fa, g, inputs, outputs, eager, seeds, fresh):
    """For each seed: new values into the captured inputs, replay, compare
    with an eager call on the same inputs (which also runs eager library work
    between the replays)."""
    for seed in seeds:
        for buf, new in zip(inputs, fresh(seed)):
            buf.copy_(new)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outputs]
        want = eager()
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a, b), "replay with inputs of seed %d differs from the eager call" % seed


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,dtype", [
    (2, 4, 1000, 1000, 128, True, "bf16"),     # the tiled prefill
    (4, 8, 1, 4096, 128, False, "bf16"),       # Nq = 1: split-KV decode with the library workspace
    (1, 2, 300, 5000, 64, False, "bf16"),      # a grid too small for the GPU: split prefill + combine
    (1, 1, 256, 256, 64, False, "f32"),        # float32 small grid: key chunks + float32 combine
    (1, 2, 200, 700, 32, True, "f32"),
])
def test_forward_in_a_graph(fa, B, H, Nq, Nk, d, causal, dtype):
    q, k, v = fa_inputs.make_qkv_device(B, H, Nq, Nk, d, dtype, seed=40, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
    g = _capture(lambda: fa.fa_fwd(q, k, v, causal=causal, out=out, lse=lse))

    def eager():
        return fa.fa_fwd(q, k, v, causal=causal)

    _replay_and_check(fa, g, (q, k, v), (out, lse), eager, (41, 42, 43),
                      lambda s: fa_inputs.make_qkv_device(B, H, Nq, Nk, d, dtype, seed=s, device=DEV))


def test_graph_survives_workspace_growth(fa):
    """A captured decode holds its stream's library workspace.  A later call
    on that stream that needs a larger workspace gets a new one; the old one
    stays allocated, so replays of the graph stay correct."""
    B, H, Nk, d = 2, 4, 1024, 128
    q, k, v = fa_inputs.make_qkv_device(B, H, 1, Nk, d, "bf16", seed=44, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, 1), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.fa_fwd(q, k, v, out=out, lse=lse)       # allocates the side stream's workspace
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fa.fa_fwd(q, k, v, out=out, lse=lse)
    torch.cuda.synchronize()
    # a decode with 32x the rows and 8x the keys on the same stream: its
    # workspace does not fit in the captured one, which is replaced
    qb, kb, vb = fa_inputs.make_qkv_device(8, 16, 1, 8192, d, "bf16", seed=45, device=DEV)
    side.wait_stream(torch.cuda.current_stream())   # the inputs were drawn on the current stream
    with torch.cuda.stream(side):
        big_out, big_lse = fa.fa_fwd(qb, kb, vb)
    torch.cuda.synchronize()
    want_o, want_l = fa.fa_fwd(qb, kb, vb)
    torch.cuda.synchronize()
    assert torch.equal(big_out, want_o) and torch.equal(big_lse, want_l)

    def eager():
        return fa.fa_fwd(q, k, v)

    _replay_and_check(fa, g, (q, k, v), (out, lse), eager, (46, 47),
                      lambda s: fa_inputs.make_qkv_device(B, H, 1, Nk, d, "bf16", seed=s, device=DEV))


def test_varlen_in_a_graph(fa):
    H, d = 4, 64
    lens = [700, 1, 333, 0, 1024, 65]
    cu = torch.tensor([0] + list(itertools.accumulate(lens)), dtype=torch.int32)
    total = int(cu[-1])
    cu_d = cu.to(DEV)

    def make(seed):
        g_ = torch.Generator().manual_seed(seed)
        return [torch.randn(total, H, d, generator=g_).to(torch.float16).to(DEV) for _ in range(3)]

    q, k, v = make(50)
    out = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(fa.fa_varlen_workspace_bytes(len(lens), total), 16), dtype=torch.uint8, device=DEV)
    g = _capture(lambda: fa.fa_fwd_varlen(q, k, v, cu_d, cu_d, causal=True, out=out, lse=lse, workspace=ws))

    def eager():
        return fa.fa_fwd_varlen(q, k, v, cu_d, cu_d, causal=True)

    _replay_and_check(fa, g, (q, k, v), (out, lse), eager, (51, 52, 53), make)


def test_backward_in_a_graph(fa):
    B, H, N, d = 1, 4, 700, 128
    q, k, v = fa_inputs.make_qkv_device(B, H, N, N, d, "bf16", seed=60, device=DEV)
    dout = fa_inputs.make_dout(B, H, N, d, "bf16", 61).to(DEV)
    out, lse = fa.fa_fwd(q, k, v, causal=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=DEV)
    g = _capture(lambda: fa.fa_bwd(q, k, v, out, dout, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws))

    def eager():
        return fa.fa_bwd(q, k, v, out, dout, lse, causal=True)

    def fresh(seed):
        nq, nk, nv = fa_inputs.make_qkv_device(B, H, N, N, d, "bf16", seed=seed, device=DEV)
        no, nl = fa.fa_fwd(nq, nk, nv, causal=True)
        nd = fa_inputs.make_dout(B, H, N, d, "bf16", seed + 100).to(DEV)
        return nq, nk, nv, no, nd, nl

    _replay_and_check(fa, g, (q, k, v, out, dout, lse), (dq, dk, dv), eager, (62, 63, 64), fresh)


def test_fp8_in_a_graph(fa):
    """Quantisation (which clears its amax words with a kernel) and the FP8
    attention captured together."""
    B, H, N, d = 1, 4, 640, 128
    q, k, v = fa_inputs.make_qkv_device(B, H, N, N, d, "bf16", seed=70, device=DEV)
    signs = fa_inputs.make_signs(d, 71).to(DEV)
    pack = torch.empty(fa.fa_fp8_pack_bytes(B, H, N, N, d), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)

    def step():
        fa.fa_quantize_fp8(q, k, v, signs=signs, pack=pack)
        fa.fa_fwd_fp8(pack, B, H, N, N, d, causal=True, out=out, lse=lse)

    g = _capture(step)

    def eager():
        p = fa.fa_quantize_fp8(q, k, v, signs=signs)
        return fa.fa_fwd_fp8(p, B, H, N, N, d, causal=True)

    _replay_and_check(fa, g, (q, k, v), (out, lse), eager, (72, 73, 74),
                      lambda s: fa_inputs.make_qkv_device(B, H, N, N, d, "bf16", seed=s, device=DEV))
