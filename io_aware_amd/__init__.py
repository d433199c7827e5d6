"""io_aware_amd -- FlashAttention forward for MI355X (gfx950).

A thin ctypes binding over ``libfa.so`` (the C ABI in ``include/fa.h``).  The
functions keep the C names and only marshal arguments: torch tensors become
device pointers and sizes, the current HIP stream becomes the ``stream``
argument, and a non-zero status becomes an ``FAError``.  Every step of the
computation runs in the library's HIP kernels; there is no other code path.
PyTorch is used only for device memory and streams.

The library is loaded at import; if it has not been built the import fails
(build it with ``python -m io_aware_amd.build``).
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_WORKSPACE = 0, 1, 2, 3, 4

# every function include/fa.h declares, with its ctypes signature
_SIGNATURES = {
    "fa_fwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                              ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                              ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa_fwd_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa_splitkv_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 5),
    "fa_fwd_splitkv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]),
    "fa_fwd_paged_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_int, ctypes.c_void_p]),
    "fa_varlen_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 2),
    "fa_fwd_varlen": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int,
                                                                                  ctypes.c_int, ctypes.c_void_p,
                                                                                  ctypes.c_size_t,
                                                                                  ctypes.c_void_p]),
    "fa_fp8_pack_bytes": (ctypes.c_size_t, [ctypes.c_int] * 5),
    "fa_quantize_fp8": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 6 + [ctypes.c_void_p, ctypes.c_size_t,
                                                                                   ctypes.c_void_p]),
    "fa_fwd_fp8": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int,
                                                                              ctypes.c_int, ctypes.c_void_p]),
    "fa_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "fa_bwd": (ctypes.c_int, [ctypes.c_void_p] * 9 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int,
                                                                           ctypes.c_int, ctypes.c_void_p,
                                                                           ctypes.c_size_t, ctypes.c_void_p]),
    "fa_default_num_splits": (ctypes.c_int, [ctypes.c_int]),
    "fa_release_workspace": (ctypes.c_int, []),
    "fa_map_workgroup": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]),
    "fa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fa_last_error": (ctypes.c_char_p, []),
    "fa_version": (ctypes.c_int, []),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("io_aware_amd: %s is not built; run `python -m io_aware_amd.build` "
                          "(hipcc for gfx950) first" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.fa_last_error().decode() or lib.fa_status_string(status).decode()
        super().__init__("%s failed (%d): %s" % (where, status, msg))


def _check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FAError(status, where)


_DTYPE_CODES = None
_RAW_STREAM = None


def _dtype_code(t) -> int:
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch
        _DTYPE_CODES = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    code = _DTYPE_CODES.get(t.dtype)
    if code is None:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return code


def _stream_handle(t, stream):
    """The HIP stream handle (an int) to enqueue on: ``stream`` if given,
    else the current stream of ``t``'s device.  The current stream is read
    through torch's raw-handle accessor (a fraction of a microsecond) where
    this torch has it, else through ``torch.cuda.current_stream``."""
    global _RAW_STREAM
    if stream is not None:
        return stream.cuda_stream
    if _RAW_STREAM is None:
        import torch
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None) or \
            (lambda index: torch.cuda.current_stream(index).cuda_stream)
    return _RAW_STREAM(t.device.index)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous device tensor" % name)
        if t.dtype != q.dtype:
            raise TypeError("q, k and v must share one dtype")
    return B, H, Nq, Nk, d


def _expect(t, name, shape, dtype, device):
    """A caller-supplied output or buffer: the library writes (or reads)
    exactly ``shape`` elements of ``dtype`` through its pointer, so it must
    be a contiguous tensor of that shape and type on ``device``."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s on %s (got %s %s on %s)"
                         % (name, dtype, tuple(shape), device, t.dtype, tuple(t.shape), t.device))


def _buffer(t, name, need, device):
    """A caller-supplied byte buffer (workspace, pack) of at least ``need``
    bytes on ``device``."""
    if t is None:
        return
    if t.device != device or not t.is_contiguous() or t.numel() * t.element_size() < need:
        raise ValueError("%s must be a contiguous tensor of at least %d bytes on %s" % (name, need, device))


def _outputs(q, out, lse, want_lse):
    import torch
    B, H, Nq, d = q.shape
    _expect(out, "out", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, H, Nq), torch.float32, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    return out, lse


def fa_fwd(q, k, v, scale=None, causal=False, out=None, lse=None, return_lse=True, stream=None):
    """O = softmax(scale * Q K^T [+ causal mask]) V and LSE for [B, H, N, d]
    tensors.  Returns (out, lse) (lse None if ``return_lse`` is False and no
    ``lse`` tensor is given).  ``scale`` defaults to 1/sqrt(d)."""
    B, H, Nq, Nk, d = _shapes(q, k, v)
    out, lse = _outputs(q, out, lse, return_lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d, float(scale),
                      1 if causal else 0, _dtype_code(q), _stream_handle(q, stream)), "fa_fwd")
    return out, lse


# bytes of the static scratch array of fa_fwd_noalloc (FA_NOALLOC_SCRATCH_BYTES)
FA_NOALLOC_SCRATCH_BYTES = 16 << 20


def fa_fwd_noalloc(q, k, v, out, lse=None, scale=None, causal=False, stream=None):
    """fa_fwd through the entry point that allocates no device memory (its
    split workspace is the library's static scratch array).  ``out`` (and
    ``lse``, if wanted) must be given.  Returns (out, lse)."""
    import torch
    B, H, Nq, Nk, d = _shapes(q, k, v)
    if out is None:
        raise ValueError("fa_fwd_noalloc writes into caller-owned outputs: pass out")
    _expect(out, "out", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, H, Nq), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib.fa_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d, float(scale),
                              1 if causal else 0, _dtype_code(q), _stream_handle(q, stream)), "fa_fwd_noalloc")
    return out, lse


def fa_splitkv_workspace_bytes(B, H, Nq, d, num_splits) -> int:
    return int(lib.fa_splitkv_workspace_bytes(B, H, Nq, d, num_splits))


def fa_fwd_splitkv(q, k, v, num_splits, scale=None, workspace=None, out=None, lse=None, return_lse=True,
                   stream=None):
    """Single-token decode (Nq == 1) with ``num_splits`` K/V chunks merged by
    logsumexp weights.  ``workspace`` is a device tensor of at least
    ``fa_splitkv_workspace_bytes`` bytes (allocated here if None)."""
    import torch
    B, H, Nq, Nk, d = _shapes(q, k, v)
    out, lse = _outputs(q, out, lse, return_lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_splitkv_workspace_bytes(B, H, Nq, d, num_splits)
    _buffer(workspace, "workspace", 0, q.device)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d, float(scale),
                              int(num_splits), _ptr(workspace), ws_bytes, _dtype_code(q),
                              _stream_handle(q, stream)), "fa_fwd_splitkv")
    return out, lse


def fa_fwd_paged_decode(q, k_cache, v_cache, block_table, seq_lens, num_splits, scale=None, workspace=None,
                        out=None, lse=None, return_lse=True, stream=None):
    """Single-token decode over a paged cache.  q [B, H, 1, d]; k_cache and
    v_cache [num_blocks, H, block_size, d]; block_table int32 [B, max_blocks];
    seq_lens int32 [B].  Returns (out [B, H, 1, d], lse [B, H])."""
    import torch
    if q.dim() != 4 or q.shape[2] != 1:
        raise ValueError("q must be [B, H, 1, d]")
    B, H, _, d = q.shape
    if k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[1] != H \
            or k_cache.shape[3] != d:
        raise ValueError("k_cache and v_cache must be [num_blocks, H, block_size, d]")
    num_blocks, _, block_size, _ = k_cache.shape
    if block_table.dim() != 2 or block_table.shape[0] != B or block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32 [B, max_blocks]")
    if seq_lens.dim() != 1 or seq_lens.shape[0] != B or seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32 [B]")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table),
                    ("seq_lens", seq_lens)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous device tensor" % name)
    _expect(out, "out", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, H), torch.float32, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_splitkv_workspace_bytes(B, H, 1, d, num_splits)
    _buffer(workspace, "workspace", 0, q.device)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.fa_fwd_paged_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                   _ptr(out), _ptr(lse), B, H, d, block_size, block_table.shape[1], num_blocks,
                                   float(scale), int(num_splits), _ptr(workspace), ws_bytes, _dtype_code(q),
                                   _stream_handle(q, stream)), "fa_fwd_paged_decode")
    return out, lse


def fa_varlen_workspace_bytes(num_seqs, total_q) -> int:
    return int(lib.fa_varlen_workspace_bytes(num_seqs, total_q))


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale=None, causal=False, out=None, lse=None,
                  return_lse=True, workspace=None, stream=None):
    """Forward over packed variable-length sequences: q [total_q, H, d],
    k and v [total_k, H, d], cu_seqlens_* int32 [S + 1] device offsets.
    Returns (out [total_q, H, d], lse [H, total_q])."""
    import torch
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or q.shape[1:] != k.shape[1:] or k.shape != v.shape:
        raise ValueError("q must be [total_q, H, d] and k, v [total_k, H, d]")
    total_q, H, d = q.shape
    total_k = k.shape[0]
    for name, t in (("q", q), ("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous device tensor" % name)
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32 or \
            cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be int32 [S + 1]")
    S = cu_seqlens_q.shape[0] - 1
    _expect(out, "out", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (H, total_q), torch.float32, q.device)
    out = torch.empty_like(q) if out is None else out
    if lse is None and return_lse:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_varlen_workspace_bytes(S, total_q)
    _buffer(workspace, "workspace", 0, q.device)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                             _ptr(cu_seqlens_k), S, total_q, total_k, H, d, float(scale), 1 if causal else 0,
                             _dtype_code(q), _ptr(workspace), ws_bytes, _stream_handle(q, stream)), "fa_fwd_varlen")
    return out, lse


def fa_fp8_pack_bytes(B, H, Nq, Nk, d) -> int:
    return int(lib.fa_fp8_pack_bytes(B, H, Nq, Nk, d))


def fa_quantize_fp8(q, k, v, signs=None, pack=None, stream=None):
    """q [B, H, Nq, d], k and v [B, H, Nk, d] (fp16 / bf16) -> the E4M3 pack
    (a uint8 device tensor of fa_fp8_pack_bytes bytes).  ``signs``: a float32
    device tensor [d] of +-1 for the incoherent transform, or None."""
    import torch
    B, H, Nq, Nk, d = _shapes(q, k, v)
    need = fa_fp8_pack_bytes(B, H, Nq, Nk, d)
    _buffer(pack, "pack", 0, q.device)
    if pack is None:
        pack = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if signs is not None and (signs.dtype != torch.float32 or signs.numel() != d or not signs.is_cuda):
        raise ValueError("signs must be a float32 device tensor of d elements")
    _check(lib.fa_quantize_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(signs), B, H, Nq, Nk, d, _dtype_code(q), _ptr(pack),
                               pack.numel() * pack.element_size(), _stream_handle(q, stream)), "fa_quantize_fp8")
    return pack


def fa_fwd_fp8(pack, B, H, Nq, Nk, d, scale=None, causal=False, out_dtype=None, out=None, lse=None,
               return_lse=True, stream=None):
    """Attention on an E4M3 pack.  Returns (out [B, H, Nq, d], lse [B, H, Nq])."""
    import torch
    # the pack is read whole: it must hold what fa_quantize_fp8 wrote for these sizes
    _buffer(pack, "pack", fa_fp8_pack_bytes(B, H, Nq, Nk, d), pack.device)
    if not pack.is_cuda:
        raise ValueError("pack must be a device tensor")
    if out is not None:
        _expect(out, "out", (B, H, Nq, d), out.dtype, pack.device)
    _expect(lse, "lse", (B, H, Nq), torch.float32, pack.device)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype or torch.bfloat16, device=pack.device)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=pack.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib.fa_fwd_fp8(_ptr(pack), _ptr(out), _ptr(lse), B, H, Nq, Nk, d, float(scale), 1 if causal else 0,
                          _dtype_code(out), _stream_handle(out, stream)), "fa_fwd_fp8")
    return out, lse


def fa_bwd_workspace_bytes(B, H, Nq, d) -> int:
    return int(lib.fa_bwd_workspace_bytes(B, H, Nq, d))


def fa_bwd(q, k, v, out, dout, lse, scale=None, causal=False, dq=None, dk=None, dv=None, workspace=None,
           stream=None):
    """Gradients (dq, dk, dv) of the forward for the upstream gradient
    ``dout``, from the forward's ``out`` and ``lse`` ([B, H, Nq] float32).
    ``workspace`` is a device tensor of at least ``fa_bwd_workspace_bytes``
    bytes (allocated here if None)."""
    import torch
    B, H, Nq, Nk, d = _shapes(q, k, v)
    for name, t in (("out", out), ("dout", dout)):
        if tuple(t.shape) != tuple(q.shape) or t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous device tensor shaped and typed like q" % name)
    _expect(lse, "lse", (B, H, Nq), torch.float32, q.device)
    _expect(dq, "dq", q.shape, q.dtype, q.device)
    _expect(dk, "dk", k.shape, k.dtype, k.device)
    _expect(dv, "dv", v.shape, v.dtype, v.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_bwd_workspace_bytes(B, H, Nq, d)
    _buffer(workspace, "workspace", 0, q.device)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                      B, H, Nq, Nk, d, float(scale), 1 if causal else 0, _dtype_code(q), _ptr(workspace), ws_bytes,
                      _stream_handle(q, stream)), "fa_bwd")
    return dq, dk, dv


def fa_default_num_splits(Nk: int) -> int:
    return int(lib.fa_default_num_splits(Nk))


def fa_release_workspace() -> None:
    _check(lib.fa_release_workspace(), "fa_release_workspace")


def fa_map_workgroup(wg: int, BH: int, Tr: int, causal: bool):
    bh, qb = ctypes.c_int(-1), ctypes.c_int(-1)
    _check(lib.fa_map_workgroup(wg, BH, Tr, 1 if causal else 0, ctypes.byref(bh), ctypes.byref(qb)),
           "fa_map_workgroup")
    return bh.value, qb.value


def fa_status_string(status: int) -> str:
    return lib.fa_status_string(status).decode()


def fa_last_error() -> str:
    return lib.fa_last_error().decode()


def fa_version() -> int:
    return int(lib.fa_version())


__all__ = ["fa_fwd", "fa_fwd_fp8", "fa_quantize_fp8", "fa_fp8_pack_bytes", "fa_fwd_varlen", "fa_varlen_workspace_bytes", "fa_bwd", "fa_bwd_workspace_bytes", "fa_fwd_splitkv", "fa_fwd_paged_decode", "fa_splitkv_workspace_bytes", "fa_default_num_splits",
           "fa_release_workspace", "fa_map_workgroup", "fa_status_string", "fa_last_error", "fa_version",
           "FAError", "FA_F32", "FA_F16", "FA_BF16", "lib", "LIB_PATH"]
