"""The C ABI on the host: the library loads, exports every function
include/fa.h declares, and rejects every invalid argument before any HIP
call (so these run without a GPU), plus the host-side planning logic.

Pointers passed here are fake, 16-byte aligned addresses: every call below is
built so that validation rejects it, and validation runs before the library
touches HIP or memory.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def fa():
    lib_path = os.path.join(ROOT, "io_aware_amd", "libfa.so")
    if not os.path.exists(lib_path):        # build once, without importing the package
        import importlib.util
        spec = importlib.util.spec_from_file_location("fa_build", os.path.join(ROOT, "io_aware_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import io_aware_amd
    return io_aware_amd


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("fa_fwd", "fa_fwd_noalloc", "fa_fwd_fp8", "fa_quantize_fp8", "fa_fp8_pack_bytes", "fa_fwd_varlen", "fa_varlen_workspace_bytes", "fa_bwd", "fa_bwd_workspace_bytes", "fa_fwd_splitkv", "fa_fwd_paged_decode", "fa_splitkv_workspace_bytes", "fa_status_string",
                 "fa_last_error", "fa_release_workspace", "fa_default_num_splits", "fa_map_workgroup"):
        assert want in names


def test_library_exports_every_declared_symbol(fa):
    names = declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(line.split()[-1] for line in out.stdout.splitlines() if line.strip())
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert getattr(fa.lib, n) is not None
    # the binding wraps every declared function under the same name
    for n in names:
        assert callable(getattr(fa, n)), n


def test_version_and_status_strings(fa):
    assert fa.fa_version() == 1
    for code in range(5):
        assert fa.fa_status_string(code).startswith(["FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED",
                                                     "FA_ERR_HIP", "FA_ERR_WORKSPACE"][code])
    assert "unknown" in fa.fa_status_string(99)


# fake device addresses: 16-byte aligned, far apart
Q, K, V, O, L, W = (0x10000000 * i for i in range(1, 7))
GOOD = dict(q=Q, k=K, v=V, out=O, lse=L, B=2, H=4, Nq=100, Nk=100, d=64, scale=0.125, causal=0, dtype=2)


def call_fwd(fa, **over):
    a = dict(GOOD)
    a.update(over)
    return fa.lib.fa_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                         a["scale"], a["causal"], a["dtype"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(out=None), 1),
    (dict(B=0), 1), (dict(H=-1), 1), (dict(Nq=0), 1), (dict(Nk=0), 1), (dict(d=0), 1),
    (dict(scale=math.nan), 1), (dict(scale=math.inf), 1), (dict(scale=-math.inf), 1), (dict(scale=3e38), 1),
    (dict(scale=-3e38), 1), (dict(causal=2), 1), (dict(causal=-1), 1),
    (dict(dtype=3), 2), (dict(dtype=-1), 2),
    (dict(d=48), 2), (dict(d=256), 2), (dict(d=16), 2),
    (dict(q=Q + 8), 2), (dict(out=O + 4), 2), (dict(lse=L + 2), 2),
    (dict(Nq=1 << 26, d=64), 2),
    (dict(B=1 << 15, H=1 << 15, Nq=1 << 20, Nk=1 << 20, d=64), 2),   # 2^56 elements: past the 2^48 cap
    (dict(out=Q + 64), 1), (dict(lse=K + 1024), 1), (dict(lse=O + 16), 1),
])
def test_fwd_rejects_invalid_arguments(fa, over, code):
    assert call_fwd(fa, **over) == code
    assert fa.fa_last_error() != ""


@pytest.mark.parametrize("scale", [-0.125, 0.0, -0.0, 1e-30, -2.3e38, 2.3e38])
def test_every_finite_scale_passes_validation(fa, scale):
    # the scale check runs before the head-dim check: an accepted scale
    # leaves the call to be rejected for d = 48 (unsupported), not for scale
    assert call_fwd(fa, scale=scale, d=48) == 2
    assert call_fwd_noalloc(fa, scale=scale, d=48) == 2
    assert "d must be" in fa.fa_last_error()
    assert call_split(fa, scale=scale, d=48) == 2
    assert call_paged(fa, scale=scale, d=48) == 2
    assert call_bwd(fa, scale=scale, d=48) == 2
    assert call_varlen(fa, scale=scale, d=48) == 2
    assert call_fwd_fp8(fa, scale=scale, dtype=0) == 2   # its size checks come first: reject the out type


def call_fwd_noalloc(fa, **over):
    a = dict(GOOD)
    a.update(over)
    return fa.lib.fa_fwd_noalloc(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"],
                                 a["d"], a["scale"], a["causal"], a["dtype"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(B=0), 1), (dict(scale=math.nan), 1), (dict(causal=2), 1), (dict(dtype=3), 2),
    (dict(d=48), 2), (dict(out=O + 4), 2), (dict(out=Q + 64), 1),
    # a decode whose one-chunk workspace, B*H*(d + 1)*4 bytes, exceeds the scratch array
    (dict(B=1024, H=64, Nq=1, Nk=1, d=128), 4),
])
def test_fwd_noalloc_rejects_invalid_arguments(fa, over, code):
    assert call_fwd_noalloc(fa, **over) == code
    assert fa.fa_last_error() != ""


def test_noalloc_scratch_size_is_the_header_constant(fa):
    text = open(HEADER).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.FA_NOALLOC_SCRATCH_BYTES
    # the decode workload (16 x 32 heads, d = 128, 32 chunks) fits it
    assert fa.fa_splitkv_workspace_bytes(16, 32, 1, 128, 32) <= fa.FA_NOALLOC_SCRATCH_BYTES


def test_error_message_is_per_thread(fa):
    import threading
    assert call_fwd(fa, d=48) == 2
    seen = {}

    def other():
        seen["msg"] = fa.fa_last_error()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "d must be" in fa.fa_last_error()


def call_split(fa, S=32, ws=W, ws_bytes=None, **over):
    a = dict(GOOD, Nq=1, Nk=8192, d=128)
    a.update(over)
    if ws_bytes is None:
        ws_bytes = fa.fa_splitkv_workspace_bytes(a["B"], a["H"], a["Nq"], a["d"], S)
    return fa.lib.fa_fwd_splitkv(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"],
                                 a["d"], a["scale"], S, ws, ws_bytes, a["dtype"], None)


def test_splitkv_rejects_invalid_arguments(fa):
    assert call_split(fa, S=0) == 1
    assert call_split(fa, S=1025) == 1
    assert call_split(fa, q=None) == 1
    assert call_split(fa, Nq=2) == 2                   # decode only
    assert call_split(fa, dtype=0) == 2                # fp16 / bf16 only
    assert call_split(fa, ws=None) == 4
    assert call_split(fa, ws=W + 8) == 4
    assert call_split(fa, ws_bytes=1024) == 4
    assert call_split(fa, ws=K) == 4                   # overlaps k


def test_workspace_bytes(fa):
    n = fa.fa_splitkv_workspace_bytes(16, 32, 1, 128, 32)
    assert n == 16 * 32 * 32 * 129 * 4                  # already a multiple of 256
    assert fa.fa_splitkv_workspace_bytes(1, 1, 1, 64, 3) == 1024   # 780 bytes rounded up to 256
    assert fa.fa_splitkv_workspace_bytes(0, 1, 1, 64, 3) == 0
    assert fa.fa_splitkv_workspace_bytes(1, 1, 1, 64, 0) == 0
    assert fa.fa_splitkv_workspace_bytes(1, 1, 1, 64, 2000) == 0


def test_default_num_splits(fa):
    assert fa.fa_default_num_splits(8192) == 32          # 32 chunks of 256 keys
    assert fa.fa_default_num_splits(1) == 1
    assert fa.fa_default_num_splits(257) == 2
    assert fa.fa_default_num_splits(10 ** 6) == 64
    assert fa.fa_default_num_splits(0) == 0


@pytest.mark.parametrize("BH,Tr", [(128, 32), (32, 128), (16, 8), (3, 5), (1, 1), (512, 1), (24, 33), (8, 3),
                                   (136, 7)])
@pytest.mark.parametrize("causal", [False, True])
def test_workgroup_order_is_a_bijection(fa, BH, Tr, causal):
    seen = set()
    for wg in range(BH * Tr):
        bh, qb = fa.fa_map_workgroup(wg, BH, Tr, causal)
        assert 0 <= bh < BH and 0 <= qb < Tr
        seen.add((bh, qb))
    assert len(seen) == BH * Tr
    with pytest.raises(fa.FAError):
        fa.fa_map_workgroup(BH * Tr, BH, Tr, causal)


def test_workgroup_order_groups_heads_by_xcd(fa):
    # 128 heads x 32 blocks: XCD x (= wg % 8) gets heads 16x .. 16x+15
    BH, Tr = 128, 32
    for wg in range(0, BH * Tr, 37):
        bh, _ = fa.fa_map_workgroup(wg, BH, Tr, True)
        assert bh // 16 == wg % 8
    # causal: the first workgroup of a head takes its last (longest) block
    assert fa.fa_map_workgroup(0, BH, Tr, True) == (0, Tr - 1)
    assert fa.fa_map_workgroup(0, BH, Tr, False) == (0, 0)


@pytest.mark.parametrize("BH,Tr", [(32, 128), (128, 32), (8, 3), (24, 33)])
def test_non_causal_order_is_one_head_at_a_time(fa, BH, Tr):
    """Without the mask every Q block has the same length: XCD x walks its
    heads one at a time, each head's blocks in order, so the blocks running
    at once share that head's K/V in the XCD's L2."""
    nwg = BH * Tr
    if nwg % 8:
        seq = [fa.fa_map_workgroup(wg, BH, Tr, False) for wg in range(nwg)]
        assert seq == [(h, b) for h in range(BH) for b in range(Tr)]
        return
    per_xcd = nwg // 8
    for x in range(8):
        seq = [fa.fa_map_workgroup(8 * w + x, BH, Tr, False) for w in range(per_xcd)]
        flat = [bh * Tr + qb for bh, qb in seq]
        assert flat == list(range(x * per_xcd, (x + 1) * per_xcd))


@pytest.mark.parametrize("BH,Tr", [(128, 32), (512, 16), (32, 128), (24, 33), (8, 3)])
def test_causal_order_phases_and_head_groups(fa, BH, Tr):
    """Causal order on each XCD: first the Q blocks >= Tr/4 four heads at a
    time (interleaved, longest first), then the blocks < Tr/4 the same way."""
    hpx = BH // 8
    gh = min(4, hpx)
    while hpx % gh:
        gh -= 1
    split = Tr // 4
    for x in range(8):
        seq = [fa.fa_map_workgroup(8 * w + x, BH, Tr, True) for w in range(hpx * Tr)]
        assert all(bh // hpx == x for bh, _ in seq)                    # whole heads per XCD
        n1 = (Tr - split) * hpx
        assert all(qb >= split for _, qb in seq[:n1]) and all(qb < split for _, qb in seq[n1:])
        for lo, hi, part in ((split, Tr, seq[:n1]), (0, split, seq[n1:])):
            if hi == lo:                                                # Tr < 4: no second phase
                assert not part
                continue
            per_group = (hi - lo) * gh
            for g0 in range(0, len(part), per_group):
                grp = part[g0:g0 + per_group]
                heads = sorted(set(bh for bh, _ in grp))
                assert len(heads) == gh and heads == list(range(heads[0], heads[0] + gh))
                blocks = [qb for _, qb in grp]
                assert blocks == sorted(blocks, reverse=True)           # longest first within the group
                assert blocks[0] == hi - 1


# fake addresses for the paged entry point: caches, table and lengths far apart
KC, VC, TB, SL = (0x10000000 * i for i in range(8, 12))
PGOOD = dict(q=Q, kc=KC, vc=VC, table=TB, lens=SL, out=O, lse=L, B=4, H=8, d=128, bs=16, max_blocks=64,
             num_blocks=256, scale=0.125, S=8, ws=W, dtype=2)


def call_paged(fa, ws_bytes=None, **over):
    a = dict(PGOOD)
    a.update(over)
    if ws_bytes is None:
        ws_bytes = fa.fa_splitkv_workspace_bytes(a["B"], a["H"], 1, a["d"], max(1, min(a["S"], 1024)))
    return fa.lib.fa_fwd_paged_decode(a["q"], a["kc"], a["vc"], a["table"], a["lens"], a["out"], a["lse"],
                                      a["B"], a["H"], a["d"], a["bs"], a["max_blocks"], a["num_blocks"],
                                      a["scale"], a["S"], a["ws"], ws_bytes, a["dtype"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(kc=None), 1), (dict(vc=None), 1), (dict(table=None), 1), (dict(lens=None), 1),
    (dict(out=None), 1), (dict(B=0), 1), (dict(H=0), 1), (dict(bs=0), 1), (dict(max_blocks=0), 1),
    (dict(num_blocks=0), 1), (dict(scale=3e38), 1), (dict(scale=math.nan), 1), (dict(S=0), 1), (dict(S=1025), 1),
    (dict(dtype=0), 2), (dict(dtype=5), 2), (dict(d=96), 2),
    (dict(bs=12), 2), (dict(bs=2048), 2),
    (dict(max_blocks=1 << 27, bs=32), 2), (dict(num_blocks=1 << 29), 2),
    (dict(q=Q + 8), 2), (dict(kc=KC + 4), 2), (dict(table=TB + 2), 2), (dict(lens=SL + 1), 2),
    (dict(lse=L + 2), 2),
    (dict(out=KC + 4096), 1), (dict(lse=TB), 1), (dict(lse=O + 16), 1), (dict(out=SL), 1),
    (dict(ws=None), 4), (dict(ws=W + 8), 4), (dict(ws=VC + 1024), 4), (dict(ws=O), 4),
])
def test_paged_decode_rejects_invalid_arguments(fa, over, code):
    assert call_paged(fa, **over) == code
    assert fa.fa_last_error() != ""


def test_paged_decode_rejects_small_workspace(fa):
    need = fa.fa_splitkv_workspace_bytes(4, 8, 1, 128, 8)
    assert call_paged(fa, ws_bytes=need - 1) == 4
    assert "workspace" in fa.fa_last_error()


BQ_, BK_, BV_, BO_, BDO_, BL_, GQ_, GK_, GV_, BW_ = (0x10000000 * i for i in range(12, 22))
BGOOD = dict(q=BQ_, k=BK_, v=BV_, out=BO_, dout=BDO_, lse=BL_, dq=GQ_, dk=GK_, dv=GV_, B=2, H=4, Nq=100, Nk=120,
             d=64, scale=0.125, causal=1, dtype=2, ws=BW_)


def call_bwd(fa, ws_bytes=None, **over):
    a = dict(BGOOD)
    a.update(over)
    if ws_bytes is None:
        ws_bytes = fa.fa_bwd_workspace_bytes(a["B"], a["H"], a["Nq"], 64)
    return fa.lib.fa_bwd(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                         a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"], a["ws"],
                         ws_bytes, None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(dout=None), 1), (dict(lse=None), 1), (dict(dq=None), 1), (dict(dk=None), 1),
    (dict(dv=None), 1), (dict(out=None), 1), (dict(B=0), 1), (dict(Nk=0), 1), (dict(scale=math.inf), 1),
    (dict(causal=3), 1),
    (dict(dtype=0), 2), (dict(d=48), 2), (dict(dout=BDO_ + 8), 2), (dict(dq=GQ_ + 8), 2), (dict(lse=BL_ + 2), 2),
    (dict(dq=BQ_ + 64), 1), (dict(dk=BV_), 1), (dict(dv=BL_), 1), (dict(dv=GK_ + 64), 1), (dict(dk=BDO_), 1),
    (dict(ws=None), 4), (dict(ws=BW_ + 8), 4), (dict(ws=BO_), 4), (dict(ws=GV_ + 16), 4),
])
def test_bwd_rejects_invalid_arguments(fa, over, code):
    assert call_bwd(fa, **over) == code
    assert fa.fa_last_error() != ""


def test_bwd_workspace_bytes(fa):
    assert fa.fa_bwd_workspace_bytes(8, 16, 4096, 128) == (8 * 16 * 4096 + 64) * 8
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 64) == 768          # 65 rows * 8 bytes = 520, rounded to 256
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 48) == 0
    assert fa.fa_bwd_workspace_bytes(0, 1, 1, 64) == 0
    assert call_bwd(fa, ws_bytes=fa.fa_bwd_workspace_bytes(2, 4, 100, 64) - 1) == 4


VQ, VK, VV, VO, VL, VCQ, VCK, VW = (0x10000000 * i for i in range(22, 30))
VGOOD = dict(q=VQ, k=VK, v=VV, out=VO, lse=VL, cq=VCQ, ck=VCK, S=4, total_q=1000, total_k=900, H=8, d=128,
             scale=0.125, causal=1, dtype=2, ws=VW)


def call_varlen(fa, ws_bytes=None, **over):
    a = dict(VGOOD)
    a.update(over)
    if ws_bytes is None:
        ws_bytes = fa.fa_varlen_workspace_bytes(max(1, min(a["S"], 4096)), max(1, a["total_q"]))
    return fa.lib.fa_fwd_varlen(a["q"], a["k"], a["v"], a["out"], a["lse"], a["cq"], a["ck"], a["S"],
                                a["total_q"], a["total_k"], a["H"], a["d"], a["scale"], a["causal"], a["dtype"],
                                a["ws"], ws_bytes, None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(cq=None), 1), (dict(ck=None), 1), (dict(out=None), 1), (dict(S=0), 1),
    (dict(total_q=0), 1), (dict(total_k=0), 1), (dict(H=0), 1), (dict(scale=-math.inf), 1), (dict(causal=2), 1),
    (dict(dtype=0), 2), (dict(d=80), 2), (dict(S=4097), 2), (dict(total_q=1 << 25), 2),
    (dict(q=VQ + 8), 2), (dict(cq=VCQ + 2), 2), (dict(lse=VL + 1), 2),
    (dict(out=VK + 64), 1), (dict(lse=VCQ), 1), (dict(lse=VO + 16), 1),
    (dict(ws=None), 4), (dict(ws=VW + 4), 4), (dict(ws=VO), 4), (dict(ws=VCK), 4),
])
def test_varlen_rejects_invalid_arguments(fa, over, code):
    assert call_varlen(fa, **over) == code
    assert fa.fa_last_error() != ""


def test_varlen_workspace_bytes(fa):
    # 4 * (2 + 2 * (ceil(1000 / 128) + 4)) = 104 -> 256
    assert fa.fa_varlen_workspace_bytes(4, 1000) == 256
    assert fa.fa_varlen_workspace_bytes(16, 70000) == ((2 + 2 * (547 + 16)) * 4 + 255) // 256 * 256
    assert fa.fa_varlen_workspace_bytes(0, 10) == 0 and fa.fa_varlen_workspace_bytes(4097, 10) == 0
    assert call_varlen(fa, ws_bytes=100) == 4


FQ, FK, FV, FS, FP, FO, FL = (0x10000000 * i for i in range(30, 37))


def call_quant(fa, pack_bytes=None, **over):
    a = dict(q=FQ, k=FK, v=FV, signs=FS, B=2, H=4, Nq=300, Nk=500, d=128, dtype=2, pack=FP)
    a.update(over)
    if pack_bytes is None:
        pack_bytes = fa.fa_fp8_pack_bytes(2, 4, 300, 500, 128)
    return fa.lib.fa_quantize_fp8(a["q"], a["k"], a["v"], a["signs"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                                  a["dtype"], a["pack"], pack_bytes, None)


def call_fwd_fp8(fa, **over):
    a = dict(pack=FP, out=FO, lse=FL, B=2, H=4, Nq=300, Nk=500, d=128, scale=0.088, causal=1, dtype=2)
    a.update(over)
    return fa.lib.fa_fwd_fp8(a["pack"], a["out"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"],
                             a["causal"], a["dtype"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(pack=None), 1), (dict(B=0), 1), (dict(Nk=0), 1),
    (dict(d=32), 2), (dict(d=96), 2), (dict(dtype=0), 2), (dict(q=FQ + 8), 2), (dict(pack=FP + 16), 2),
    (dict(signs=FS + 2), 2), (dict(pack=FK), 1), (dict(pack=FQ + 256), 1),
])
def test_quantize_fp8_rejects_invalid_arguments(fa, over, code):
    assert call_quant(fa, **over) == code
    assert fa.fa_last_error() != ""


@pytest.mark.parametrize("over,code", [
    (dict(pack=None), 1), (dict(out=None), 1), (dict(H=0), 1), (dict(scale=math.nan), 1), (dict(causal=5), 1),
    (dict(d=32), 2), (dict(dtype=0), 2), (dict(pack=FP + 64), 2), (dict(out=FO + 8), 2), (dict(lse=FL + 1), 2),
    (dict(out=FP + 1024), 1), (dict(lse=FO + 16), 1),
])
def test_fwd_fp8_rejects_invalid_arguments(fa, over, code):
    assert call_fwd_fp8(fa, **over) == code
    assert fa.fa_last_error() != ""


def test_fp8_pack_bytes_follow_the_documented_layout(fa):
    up = lambda x: (x + 255) // 256 * 256
    B, H, Nq, Nk, d = 2, 4, 300, 500, 128
    BH, Nkp = B * H, 512
    want = up(BH * Nq * d) + up(BH * Nkp * d) + up(BH * d * Nkp) + 2 * up(3 * BH * 4)
    assert fa.fa_fp8_pack_bytes(B, H, Nq, Nk, d) == want
    assert fa.fa_fp8_pack_bytes(B, H, Nq, Nk, 32) == 0
    assert call_quant(fa, pack_bytes=want - 1) == 4


def test_binding_checks_caller_outputs(fa):
    # the library writes through an output pointer without knowing its size:
    # the binding accepts only a contiguous tensor of the exact shape and type
    import torch
    cpu = torch.device("cpu")
    good = torch.empty((2, 3, 5), dtype=torch.float32)
    fa._expect(good, "lse", (2, 3, 5), torch.float32, cpu)
    fa._expect(None, "lse", (2, 3, 5), torch.float32, cpu)
    for bad in (torch.empty((2, 3, 4), dtype=torch.float32),             # too small
                torch.empty((2, 3, 6), dtype=torch.float32),             # wrong shape
                torch.empty((2, 3, 5), dtype=torch.float16),             # wrong type
                torch.empty((2, 5, 3), dtype=torch.float32).transpose(1, 2)):   # strided
        with pytest.raises(ValueError):
            fa._expect(bad, "lse", (2, 3, 5), torch.float32, cpu)
    with pytest.raises(ValueError):
        fa._expect(good, "lse", (2, 3, 5), torch.float32, torch.device("cuda", 0))
    fa._buffer(torch.empty(64, dtype=torch.uint8), "workspace", 64, cpu)
    with pytest.raises(ValueError):
        fa._buffer(torch.empty(63, dtype=torch.uint8), "workspace", 64, cpu)
    with pytest.raises(ValueError):
        fa._buffer(torch.empty(64, dtype=torch.uint8), "workspace", 0, torch.device("cuda", 0))
