"""FP8 attention with incoherent processing, as the oracle computes it.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"9.4 FlashAttention 与 FlashMLA" (section 9.4.4, the FlashAttention-3
comparison) describes the FP8 mode: Q, K and V in an 8-bit float (E4M3), with
the quantisation error of Q and K spread evenly by a random orthogonal
transform applied to both ("incoherent processing").  The page fixes neither
the transform nor the scaling; the readings taken here:

* the transform is M = diag(s) H_d / sqrt(d), each row x going to x M: the
  signs s (random, +-1, drawn by the caller and passed in) first, then the
  Sylvester-Hadamard matrix H_d.  The
  same M goes to Q and K, so (Q M)(K M)^T = Q K^T and the scores are
  unchanged before rounding.  V is not transformed;
* one scale per (batch, head) and tensor: amax = max |x| over the head,
  codes = RNE_e4m3(clamp(x * (448 / amax), -448, 448)), dequantised value =
  code * (amax / 448) (448 is the largest E4M3 value);
* attention then runs on the dequantised Q', K', V exactly (``attention``).

The quantised codes are integers decided by float32 arithmetic, so this
module takes those decisions in float32, in the order the library's kernel
takes them (the butterfly of the fast Walsh-Hadamard transform stage by
stage, then one multiply by fp32(1/sqrt(d)); the scale 448/amax as one
float32 division; one multiply; the E4M3 rounding).  Everything after the
codes is fp64.
"""
from __future__ import annotations

import numpy as np
import torch

from . import attention

E4M3_MAX = 448.0


def fwht_f32(x) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis in
    float32: for h = 1, 2, 4, ..., d/2, each pair (i, i + h) with bit h of i
    clear becomes (x_i + x_{i+h}, x_i - x_{i+h}).  Equals x @ H_d (H_d the
    Sylvester-Hadamard matrix) up to float32 rounding."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("d must be a power of two")
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def incoherent_transform(x, signs) -> np.ndarray:
    """x -> (x * signs) H_d / sqrt(d) along the last axis, in float32 (the
    sign flip is exact, the butterfly rounds per stage, then one multiply by
    fp32(1/sqrt(d)))."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    s = np.asarray(signs, dtype=np.float32)
    y = fwht_f32(x * s)
    return y * np.float32(1.0 / np.sqrt(d))


def to_e4m3_codes(x) -> np.ndarray:
    """float32 -> E4M3 (OCP, no infinities, max 448) with round-to-nearest-
    even, as uint8 codes; |x| must not exceed 448."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_values(codes) -> np.ndarray:
    """E4M3 codes -> float64 values."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def quantize_heads(x):
    """Per-(batch, head) E4M3 quantisation of x [B, H, N, d] (float32).

    Returns (codes uint8 [B, H, N, d], descale float32 [B, H]) with
    descale = amax / 448 (1 for an all-zero head) and codes =
    RNE(clamp(x * (448 / amax), -448, 448))."""
    x = np.asarray(x, dtype=np.float32)
    B, H = x.shape[:2]
    amax = np.abs(x).reshape(B, H, -1).max(axis=2).astype(np.float32)
    pos = amax > 0
    inv = np.where(pos, np.float32(E4M3_MAX) / np.where(pos, amax, 1), np.float32(1)).astype(np.float32)
    descale = np.where(pos, amax / np.float32(E4M3_MAX), np.float32(1)).astype(np.float32)
    y = (x * inv[:, :, None, None]).astype(np.float32)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    return to_e4m3_codes(y), descale


def quantize_qkv(q, k, v, signs=None):
    """The quantisation step: transform Q and K (if ``signs`` is given),
    quantise Q, K, V per head.  Inputs [B, H, N, d] (any float type, widened
    exactly to float32).  Returns dict(q8, k8, v8 codes, dq, dk, dv
    descales, qt, kt the transformed float32 Q and K)."""
    f = lambda t: (t.detach().to("cpu", torch.float32).numpy() if hasattr(t, "detach")
                   else np.asarray(t, dtype=np.float32))
    qf, kf, vf = f(q), f(k), f(v)
    if signs is not None:
        qf = incoherent_transform(qf, signs)
        kf = incoherent_transform(kf, signs)
    q8, dq = quantize_heads(qf)
    k8, dk = quantize_heads(kf)
    v8, dv = quantize_heads(vf)
    return dict(q8=q8, k8=k8, v8=v8, dq=dq, dk=dk, dv=dv, qt=qf, kt=kf)


def dequantize(codes, descale) -> np.ndarray:
    """codes [B, H, N, d] and descale [B, H] -> float64 values."""
    return e4m3_values(codes) * np.asarray(descale, dtype=np.float64)[:, :, None, None]


def fp8_attention(q, k, v, scale: float, causal: bool, signs=None, rows=None, threads: int = 0):
    """Exact attention (fp64) on the quantised inputs: with Q' = q8 dq,
    K' = k8 dk, V' = v8 dv (codes times per-head descales), the scores are
    scale * dq * dk * (q8 . k8) and O = dv * softmax(.) v8, so the oracle
    runs ``attention`` on the E4M3 code values (exact in float32) with the
    scale scale*dq*dk (in double) and multiplies O by dv.  ``rows`` selects
    flat query rows as in ``attention``.  Returns (out, lse, quant), out and
    lse [B, H, Nq(, d)] (NaN where not computed)."""
    qu = quantize_qkv(q, k, v, signs)
    B, H = qu["q8"].shape[:2]
    out = None
    lse = None
    for b in range(B):
        for h in range(H):
            qc = e4m3_values(qu["q8"][b:b + 1, h:h + 1]).astype(np.float32)
            kc = e4m3_values(qu["k8"][b:b + 1, h:h + 1]).astype(np.float32)
            vc = e4m3_values(qu["v8"][b:b + 1, h:h + 1]).astype(np.float32)
            s_bh = float(scale) * float(qu["dq"][b, h]) * float(qu["dk"][b, h])
            r = None
            if rows is not None:
                Nq = qc.shape[2]
                r = [i for i in rows if (b * H + h) * Nq <= i < (b * H + h + 1) * Nq]
                if not r:
                    continue
                r = np.asarray(r, dtype=np.int64) - (b * H + h) * Nq
            o, l = attention(qc, kc, vc, s_bh, causal, rows=r, threads=threads)
            o = o * float(qu["dv"][b, h])
            if out is None:
                Nq, d = qc.shape[2], qc.shape[3]
                out = np.full((B, H, Nq, d), np.nan)
                lse = np.full((B, H, Nq), np.nan)
            if r is None:
                out[b, h] = o[0, 0]
                lse[b, h] = l[0, 0]
            else:
                out[b, h, r] = o
                lse[b, h, r] = l
    return out, lse, qu
