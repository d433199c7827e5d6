"""Plain fp64 CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import this package.  It shares no
code with the HIP library in ``io_aware_amd`` and never imports it; the
library's product path never imports this package.

Two parts:

* ``attention`` -- the parity oracle: a C program (``attn_oracle.c``) that
  computes, per query row, the three-pass safe softmax (max; sum of
  exp(x - m); normalise) of the scaled scores and the weighted sum of value
  rows, in IEEE double, with the causal mask M_ij = 0 for j <= i and -inf
  otherwise, and returns O and LSE = m + ln(l).  Sources: "6. FlashAttention
  分块逻辑" (lowentro.cn) sections 1.1 and 4.1; "9.4 FlashAttention 与
  FlashMLA" (llm-fullstack-book) sections 9.4.2 and 9.4.5.
* ``attention_bwd`` -- the gradients dQ, dK, dV of exact attention for an
  upstream gradient dO (``attn_bwd_oracle.c``): P from the three-pass
  definition, dV = P^T dO, dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D),
  dQ = scale dS K, dK = scale dS^T Q, in IEEE double.  Sources: "6.
  FlashAttention 分块逻辑" section 7.1; "9.4 FlashAttention 与 FlashMLA"
  section 9.4.5.
* ``paged_decode`` -- single-token attention over a paged K/V cache: the keys
  a sequence's block table maps (unallocated blocks dropped) are gathered in
  logical order into a contiguous K/V, which ``attention`` then takes.
  Source: "6. FlashAttention 分块逻辑" section 12.
* ``varlen_attention`` -- attention over a batch of packed sequences of
  different lengths: each sequence, cut out of the packed tensors by its
  cumulative offsets, goes through ``attention`` on its own.  Source: "9.4
  FlashAttention 与 FlashMLA" section 9.4.6 (variable-length batches).
* ``oracle.fp8`` -- the FP8 mode: incoherent processing (a random
  orthogonal transform of Q and K), per-head E4M3 quantisation in float32,
  then exact attention on the dequantised values.  Source: "9.4
  FlashAttention 与 FlashMLA" section 9.4.4.
* ``oracle.algorithms`` -- the pages' algorithms (one-pass online softmax,
  blocked forward with deferred or per-step normalisation, split-KV partials
  and their merge) in numpy fp64.  They exist to pin ``attention`` and each
  other from several independent directions; they are not the parity oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "attn_oracle.c"), os.path.join(_HERE, "attn_bwd_oracle.c")]
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``attn_oracle.c`` into ``liboracle.so`` with gcc -O2 -fopenmp.

    No -ffast-math: the oracle relies on IEEE double semantics.
    """
    global _lib
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-std=c99", "-Wall", "-shared", "-fPIC"] + _SRCS + ["-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_attention_rows.restype = ctypes.c_int
    lib.oracle_attention_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_double, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_attention_bwd.restype = ctypes.c_int
    lib.oracle_attention_bwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_double, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_default_threads.restype = ctypes.c_int
    lib.oracle_default_threads.argtypes = []
    _lib = lib
    return lib


def default_threads() -> int:
    """OpenMP threads the oracle uses when none are requested."""
    return int(_load().oracle_default_threads())


def _as_f32(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: widen exactly to float32 on the host
        import torch
        x = x.detach().to("cpu", torch.float32).numpy()
    a = np.ascontiguousarray(x, dtype=np.float32)
    return a


def attention(q, k, v, scale: float, causal: bool, rows=None, threads: int = 0):
    """Exact attention in fp64 for [B, H, N, d] inputs.

    ``q``, ``k``, ``v`` are float32-representable arrays (numpy or torch;
    bf16/fp16 tensors are widened exactly).  ``scale`` is used as given
    (pass the same float32 value the GPU receives).  ``rows`` selects flat
    query rows ``(b*H + h)*Nq + i``; None means all rows.

    Returns ``(out, lse)``: with ``rows`` None, out is [B, H, Nq, d] and lse
    [B, H, Nq]; otherwise out is [len(rows), d] and lse [len(rows)].  Both
    float64.
    """
    qa, ka, va = _as_f32(q), _as_f32(k), _as_f32(v)
    if qa.ndim != 4 or ka.ndim != 4 or va.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = qa.shape
    Nk = ka.shape[2]
    if ka.shape != (B, H, Nk, d) or va.shape != ka.shape:
        raise ValueError("shape mismatch: q %s k %s v %s" % (qa.shape, ka.shape, va.shape))
    if rows is None:
        nrows = B * H * Nq
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.size
    out = np.empty((nrows, d), dtype=np.float64)
    lse = np.empty((nrows,), dtype=np.float64)
    rc = _load().oracle_attention_rows(
        qa.ctypes.data, ka.ctypes.data, va.ctypes.data,
        B, H, Nq, Nk, d, float(scale), 1 if causal else 0,
        None if rows_arr is None else rows_arr.ctypes.data, nrows,
        out.ctypes.data, lse.ctypes.data, int(threads))
    if rc != 0:
        raise RuntimeError("oracle_attention_rows failed with code %d" % rc)
    if rows is None:
        return out.reshape(B, H, Nq, d), lse.reshape(B, H, Nq)
    return out, lse


def visible_keys(Nq: int, Nk: int, causal: bool, rows) -> np.ndarray:
    """Number of keys each flat query row sees (top-left causal alignment)."""
    i = np.asarray(rows, dtype=np.int64) % Nq
    if not causal:
        return np.full(i.shape, Nk, dtype=np.int64)
    return np.minimum(i + 1, Nk)


def paged_gather_index(block_table, seq_len: int, block_size: int, num_blocks: int):
    """(physical block, row in block) of each key a sequence sees, in logical
    order ("6. FlashAttention 分块逻辑", section 12.2).

    Logical block j of the sequence holds its keys [j*block_size,
    (j+1)*block_size); the table row maps it to a physical block.  A negative
    entry marks an unallocated block, whose keys are skipped; an entry
    >= num_blocks is taken as unallocated too (it names no block of the
    cache).  Only the first min(block_size, seq_len - j*block_size) rows of
    the last block hold keys.  ``seq_len`` is clamped to [0, len(row) *
    block_size].
    """
    row = np.asarray(block_table, dtype=np.int64).reshape(-1)
    n = max(0, min(int(seq_len), row.size * block_size))
    blks, offs = [], []
    for j in range(-(-n // block_size)):
        phys = int(row[j])
        if phys < 0 or phys >= num_blocks:
            continue
        valid = min(block_size, n - j * block_size)
        blks.extend([phys] * valid)
        offs.extend(range(valid))
    return np.array(blks, dtype=np.int64), np.array(offs, dtype=np.int64)


def paged_decode(q, k_cache, v_cache, block_table, seq_lens, scale: float, seqs=None, threads: int = 0):
    """Exact single-token attention over a paged cache, in fp64.

    q: [B, H, 1, d]; k_cache, v_cache: [num_blocks, H, block_size, d];
    block_table: [B, max_blocks] integers; seq_lens: [B].  Each sequence's
    keys (``paged_gather_index``) are gathered into K_b, V_b of shape
    [1, H, n_b, d] and passed with q[b] to ``attention``.  A sequence with no
    key gets O = 0 and LSE = -inf.  ``seqs`` selects sequences (all if None).

    Returns (out [len(seqs), H, d], lse [len(seqs), H]), float64.
    """
    num_blocks, H, block_size, d = tuple(k_cache.shape)
    table = np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table, dtype=np.int64)
    lens = np.asarray(seq_lens.cpu() if hasattr(seq_lens, "cpu") else seq_lens, dtype=np.int64).reshape(-1)
    B = table.shape[0]
    seqs = list(range(B)) if seqs is None else [int(s) for s in seqs]
    out = np.zeros((len(seqs), H, d), dtype=np.float64)
    lse = np.full((len(seqs), H), -np.inf, dtype=np.float64)
    for i, b in enumerate(seqs):
        blks, offs = paged_gather_index(table[b], int(lens[b]), block_size, num_blocks)
        if blks.size == 0:
            continue
        if hasattr(k_cache, "detach"):
            import torch
            bi, oi = torch.from_numpy(blks), torch.from_numpy(offs)
        else:
            bi, oi = blks, offs
        # [n, H, d] -> [1, H, n, d]
        kb = _as_f32(k_cache[bi, :, oi, :]).transpose(1, 0, 2)[None]
        vb = _as_f32(v_cache[bi, :, oi, :]).transpose(1, 0, 2)[None]
        qb = _as_f32(q[b:b + 1])
        o, l = attention(qb, np.ascontiguousarray(kb), np.ascontiguousarray(vb), scale, False, threads=threads)
        out[i] = o[0, :, 0, :]
        lse[i] = l[0, :, 0]
    return out, lse


def attention_bwd(q, k, v, dout, scale: float, causal: bool, heads=None, q_idx=None, k_idx=None,
                  threads: int = 0, with_delta: bool = False):
    """Exact gradients of attention in fp64 for [B, H, N, d] inputs.

    ``heads`` selects flat (b*H + h) heads (all if None); ``q_idx`` the query
    indices within a head whose dQ is wanted (all if None); ``k_idx`` the key
    indices for dK and dV (all if None).  Returns (dq, dk, dv) shaped
    [nheads, nq, d], [nheads, nk, d], [nheads, nk, d] -- reshaped to
    [B, H, N, d] when all three selections are None -- and, with
    ``with_delta``, D_i = dO_i . O_i as [nheads, Nq] ([B, H, Nq]).
    """
    qa, ka, va, ga = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dout)
    B, H, Nq, d = qa.shape
    Nk = ka.shape[2]
    if ka.shape != (B, H, Nk, d) or va.shape != ka.shape or ga.shape != qa.shape:
        raise ValueError("shape mismatch")
    sel = [None if x is None else np.ascontiguousarray(x, dtype=np.int64) for x in (heads, q_idx, k_idx)]
    nh = B * H if sel[0] is None else sel[0].size
    nq = Nq if sel[1] is None else sel[1].size
    nk = Nk if sel[2] is None else sel[2].size
    dq = np.empty((nh, nq, d), dtype=np.float64)
    dk = np.empty((nh, nk, d), dtype=np.float64)
    dv = np.empty((nh, nk, d), dtype=np.float64)
    delta = np.empty((nh, Nq), dtype=np.float64)
    ptr = [None if x is None else x.ctypes.data for x in sel]
    rc = _load().oracle_attention_bwd(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, ga.ctypes.data,
                                      B, H, Nq, Nk, d, float(scale), 1 if causal else 0,
                                      ptr[0], nh, ptr[1], nq, ptr[2], nk,
                                      dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, delta.ctypes.data,
                                      int(threads))
    if rc != 0:
        raise RuntimeError("oracle_attention_bwd failed with code %d" % rc)
    if all(x is None for x in sel):
        dq, dk, dv = dq.reshape(B, H, Nq, d), dk.reshape(B, H, Nk, d), dv.reshape(B, H, Nk, d)
        delta = delta.reshape(B, H, Nq)
    return (dq, dk, dv, delta) if with_delta else (dq, dk, dv)


def varlen_attention(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool, seqs=None, rows=None,
                     threads: int = 0):
    """Exact attention over packed variable-length sequences, in fp64.

    q: [total_q, H, d]; k, v: [total_k, H, d] (token-major, heads inside);
    cu_seqlens_q, cu_seqlens_k: [S + 1] non-decreasing offsets starting at 0.
    Sequence s is q[cu_q[s]:cu_q[s+1]] attending to k, v[cu_k[s]:cu_k[s+1]]
    with ``attention`` (causal: top-left within the sequence).  A query with
    no key gets O = 0 and LSE = -inf.  ``seqs`` restricts the work to some
    sequences (the other rows of the result stay NaN); ``rows`` maps a
    sequence to the query indices within it to compute (all if absent).

    Returns (out [total_q, H, d], lse [H, total_q]), float64.
    """
    qa, ka, va = _as_f32(q), _as_f32(k), _as_f32(v)
    cq = np.asarray(cu_seqlens_q.cpu() if hasattr(cu_seqlens_q, "cpu") else cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k.cpu() if hasattr(cu_seqlens_k, "cpu") else cu_seqlens_k, dtype=np.int64)
    total_q, H, d = qa.shape
    S = cq.size - 1
    out = np.full((total_q, H, d), np.nan)
    lse = np.full((H, total_q), np.nan)
    for s in (range(S) if seqs is None else seqs):
        a, b = int(cq[s]), int(cq[s + 1])
        ka_, kb_ = int(ck[s]), int(ck[s + 1])
        if b <= a:
            continue
        if kb_ <= ka_:
            out[a:b] = 0.0
            lse[:, a:b] = -np.inf
            continue
        qs = np.ascontiguousarray(qa[a:b].transpose(1, 0, 2))[None]      # [1, H, n, d]
        ks = np.ascontiguousarray(ka[ka_:kb_].transpose(1, 0, 2))[None]
        vs = np.ascontiguousarray(va[ka_:kb_].transpose(1, 0, 2))[None]
        if rows is not None and s in rows:
            n = b - a
            ri = np.asarray(rows[s], dtype=np.int64)
            flat = (np.arange(H, dtype=np.int64)[:, None] * n + ri[None, :]).reshape(-1)   # head-major
            o, l = attention(qs, ks, vs, scale, causal, rows=flat, threads=threads)
            o = o.reshape(H, ri.size, d)
            l = l.reshape(H, ri.size)
            out[a + ri] = o.transpose(1, 0, 2)
            lse[:, a + ri] = l
            continue
        o, l = attention(qs, ks, vs, scale, causal, threads=threads)
        out[a:b] = o[0].transpose(1, 0, 2)
        lse[:, a:b] = l[0]
    return out, lse
