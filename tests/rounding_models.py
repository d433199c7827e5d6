"""CPU models of the kernels' rounding points, for deriving parity bars.

TEST INFRASTRUCTURE.  Each model follows, in float32 torch arithmetic on the
CPU, the points where the library's kernels round: the products they form
on the matrix core (exact products of 16-bit or E4M3 inputs, float32
sums), the exponentials, the roundings of P (and dS) to the input type, the
running sums, and the final rounding of the outputs.  The models share no
code with the HIP library; they exist so that the tolerances of the GPU
parity tests can be recomputed from committed code (tests/test_models.py)
instead of being quoted.

What is modelled, and what is not:
* products: the float32 matmul of the exactly widened 16-bit (or E4M3)
  values; the matrix core's internal summation order is not reproduced
  (its effect is at float32 rounding level, far below the 16-bit effects);
* exp2 and log2 are torch's float32 functions, the hardware's are within an
  ulp or two of them;
* the lazy rescale of the forward kernels is followed per wave of 32
  queries: the accumulator is rescaled to the exact running max only when
  some query of the wave has no max yet or some lane's partial sum of P
  (the keys whose index has bit 2 equal to the lane half) exceeds the bound,
  as the kernels decide it; otherwise P is formed against the held max;
* the split prefill path for small grids is not modelled (none of the
  modelled workloads takes it).
"""
from __future__ import annotations

import numpy as np
import torch

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453
TYPES = {"bf16": torch.bfloat16, "f16": torch.float16}
NEG_INF = float("-inf")


def fma32(a, b, c):
    """float32 a * b + c with one rounding: a*b of two float32 is exact in
    float64, and the float64 sum is then rounded once more to float32."""
    return (a.double() * b.double() + c.double()).float()


def _half_masks(k0: int, n: int):
    """Which keys of a tile a lane half sums: key index bit 2 (the half that
    holds S^T register rows 8*(r >> 2) + 4*g + (r & 3))."""
    idx = torch.arange(k0, k0 + n)
    g1 = ((idx >> 2) & 1).bool()
    return (~g1).float(), g1.float()


def forward_model(q, k, v, scale: float, causal: bool, waves, *, p_type, bc: int, bound: float,
                  br: int = 128, c=None, out_type=None, out_scale=1.0, running=None):
    """The tiled forward with the lazy rescale and the rounded-P row sum
    for the 32-query waves ``waves`` of one head.

    q [Nq, d], k and v [Nk, d]: float32 tensors holding the values the
    kernel multiplies (16-bit values, or E4M3 code values).  p_type: the
    type P is rounded to before P V (torch.bfloat16, torch.float16 or
    torch.float8_e4m3fn).  bc: keys per tile; bound: the lazy-rescale bound
    on a lane's partial sum of the tile, or with ``running`` (default: for
    a bf16 P) on the lane's running sum since the last exact step, which
    bounds the accumulator as well; br: queries per workgroup (the causal
    key range ends at the workgroup's last query); c: the float32 exp2
    factor (default scale * log2 e); out_scale: multiplies O before the
    final rounding to out_type (the FP8 kernel's descale of V).

    Returns (O rounded to out_type as float64, O before that rounding as
    float64, LSE float64), each for the rows 32*w .. 32*w + 31 of every
    wave w, in that order; rows past Nq are dropped.
    """
    Nq, d = q.shape
    Nk = k.shape[0]
    out_type = out_type or p_type
    running = (p_type == torch.bfloat16) if running is None else running
    c = torch.tensor(np.float32(scale * LOG2E) if c is None else np.float32(c), dtype=torch.float32)
    W = len(waves)
    rows = torch.tensor([[32 * w + i for i in range(32)] for w in waves], dtype=torch.long)
    qr = q[rows.clamp(max=Nq - 1)]
    S = torch.matmul(qr, k.T)                                  # [W, 32, Nk] float32
    q0 = (rows[:, 0] // br) * br
    kv_end = torch.clamp(q0 + br, max=Nk) if causal else torch.full((W,), Nk)
    m = torch.full((W, 32), NEG_INF)
    l = torch.zeros((W, 32, 2))
    lt = torch.zeros((W, 32))
    acc = torch.zeros((W, 32, d))
    for k0 in range(0, int(kv_end.max()), bc):
        n = min(bc, Nk - k0)
        active = k0 < kv_end
        if causal:
            active &= k0 <= rows[:, 0] + 31
        if not bool(active.any()):
            continue
        s = S[:, :, k0:k0 + n].clone()
        if causal:
            keys = torch.arange(k0, k0 + n)
            s = torch.where(keys[None, None, :] > rows[:, :, None], torch.tensor(NEG_INF), s)
        h0, h1 = _half_masks(k0, n)

        def exp_tile(msub):
            p = torch.exp2(fma32(s, c, -msub[:, :, None]))
            return p, torch.stack([(p * h0).sum(-1), (p * h1).sum(-1)], dim=-1)

        held = torch.where(torch.isinf(m), torch.zeros_like(m), m)
        p, lh = exp_tile(held)
        test = l + lh if running else lh
        exact = torch.isinf(m).any(dim=1) | (~(test <= bound)).any(dim=2).any(dim=1)
        mx = s.max(dim=-1).values
        m_new = torch.maximum(m, mx * c)
        alpha = torch.where(torch.isinf(m_new), torch.ones_like(m_new), torch.exp2(m - m_new))
        p2, lh2 = exp_tile(torch.where(torch.isinf(m_new), torch.zeros_like(m_new), m_new))
        sel = (exact & active)[:, None]
        m = torch.where(sel, m_new, m)
        l = torch.where(sel[..., None], l * alpha[..., None], l)
        lt = torch.where(sel, lt * alpha, lt)
        acc = torch.where(sel[..., None], acc * alpha[..., None], acc)
        p = torch.where(sel[..., None], p2, p)
        lh = torch.where(sel[..., None], lh2, lh)
        act = active[:, None]
        pr = p.to(p_type).float()
        l = l + torch.where(act[..., None], lh, torch.zeros_like(lh))
        acc = acc + torch.where(act[..., None], torch.matmul(pr, v[k0:k0 + n]), torch.zeros_like(acc))
        lt = lt + torch.where(act, pr.sum(-1), torch.zeros_like(lt))
    ltot = l.sum(-1)
    inv = torch.where((ltot > 0) & (lt > 0), 1.0 / lt, torch.zeros_like(lt))
    if out_scale != 1.0:   # FP8: one factor descale_v / l8
        inv = torch.where((ltot > 0) & (lt > 0), torch.tensor(np.float32(out_scale)) / lt, torch.zeros_like(lt))
    o_pre = acc * inv[..., None]
    o = o_pre.to(out_type)
    lse = torch.where(ltot > 0, (m + torch.log2(ltot)) * np.float32(LN2), torch.tensor(NEG_INF))
    keep = (rows < Nq).reshape(-1)
    flat = lambda t: t.reshape((W * 32,) + t.shape[2:])[keep].double().numpy()
    return flat(o.float()), flat(o_pre), flat(lse)


def backward_model(q, k, v, o, lse, dout, scale: float, causal: bool, dtype: str):
    """The two backward kernels' arithmetic for one head: P rebuilt from the
    float32 LSE (times log2 e), dP = dO V^T, D = rowsum(dO * O) from the
    stored 16-bit O, dS = P (dP - D); P and dS rounded to the input type
    before their products; dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K
    accumulated in float32 and rounded to the input type.

    q, o, dout [Nq, d]; k, v [Nk, d]: float32 tensors holding 16-bit values
    (o the forward's rounded output); lse [Nq] float32.  Returns (dq, dk,
    dv) as float64 numpy arrays."""
    t = TYPES[dtype]
    Nq, d = q.shape
    Nk = k.shape[0]
    c = torch.tensor(np.float32(scale * LOG2E))
    S = torch.matmul(q, k.T)
    if causal:
        S = torch.where(torch.arange(Nk)[None, :] > torch.arange(Nq)[:, None], torch.tensor(NEG_INF), S)
    lse2 = lse.float() * np.float32(LOG2E)
    P = torch.exp2(fma32(S, c, -lse2[:, None]))
    dP = torch.matmul(dout, v.T)
    D = (dout * o).sum(-1)
    dS = P * (dP - D[:, None])
    Pr, dSr = P.to(t).float(), dS.to(t).float()
    sc = np.float32(scale)
    dv = torch.matmul(Pr.T, dout).to(t)
    dk = (torch.matmul(dSr.T, q) * sc).to(t)
    dq = (torch.matmul(dSr, k) * sc).to(t)
    return tuple(x.double().numpy() for x in (dq, dk, dv))


def grad_errors(x, ref):
    """(max |x - ref| / (|ref| + rms(ref)), mean |x - ref| / rms(ref)): the
    two figures the backward parity bar is stated in."""
    err = np.abs(x - ref)
    rms = float(np.sqrt((ref ** 2).mean()))
    return float((err / (np.abs(ref) + rms)).max()), float(err.mean() / rms)
