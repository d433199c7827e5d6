"""The pages' softmax/attention algorithms in numpy fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  These functions take
the algorithms' steps in the order the pages give them, so that the tests can
pin the three-pass oracle from independent directions: the one-pass online
recurrence must equal the three-pass softmax; the blocked forward (deferred
or per-step normalisation) must equal the unblocked definition; the split-KV
partials merged by the online rule must equal unsplit attention.

Every array is float64.  Single-head functions take Q [Nq, d], K and V
[Nk, d].  Causal masking is top-left: key j is visible to query i iff j <= i.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


# --------------------------------------------------------------------------
# 1-D softmax
# --------------------------------------------------------------------------

def softmax_three_pass(x) -> np.ndarray:
    """Safe softmax by three traversals: the max m, the sum l of exp(x - m),
    then exp(x - m) / l.  ("6. FlashAttention 分块逻辑", section 1.1.)"""
    x = np.asarray(x, dtype=np.float64)
    m = NEG_INF
    for xi in x:                      # pass 1
        if xi > m:
            m = xi
    if m == NEG_INF:
        return np.zeros_like(x)
    l = 0.0
    for xi in x:                      # pass 2
        l += math.exp(xi - m)
    return np.array([math.exp(xi - m) / l for xi in x])   # pass 3


def online_softmax_stats(x):
    """One traversal keeping the running max m and the running sum l.

    For a new element x_{k+1}: m_{k+1} = max(m_k, x_{k+1}) and
    l_{k+1} = l_k * exp(m_k - m_{k+1}) + exp(x_{k+1} - m_{k+1}); when the max
    does not move the scale factor is 1 and the step is a plain addition.
    ("6. FlashAttention 分块逻辑", section 1.2, where this is proved equal to
    the sum taken against the final max.)

    An element equal to -inf contributes exp(-inf) = 0 and leaves (m, l)
    unchanged; this also keeps m = -inf from producing -inf - (-inf).
    """
    m, l = NEG_INF, 0.0
    for xi in np.asarray(x, dtype=np.float64):
        if xi == NEG_INF:
            continue
        m_new = xi if xi > m else m
        l = l * math.exp(m - m_new) + math.exp(xi - m_new)
        m = m_new
    return m, l


def online_softmax(x) -> np.ndarray:
    """Softmax from the one-pass statistics, normalised once at the end."""
    x = np.asarray(x, dtype=np.float64)
    m, l = online_softmax_stats(x)
    if m == NEG_INF:
        return np.zeros_like(x)
    return np.exp(x - m) / l


def blockwise_softmax_stats(x, block: int):
    """The block form of the recurrence: each block's local max and local sum,
    merged into the global (m, l) with exp(m_old - m_new) and
    exp(m_local - m_new).  ("9.4 FlashAttention 与 FlashMLA", section 9.4.2.)"""
    x = np.asarray(x, dtype=np.float64)
    m, l = NEG_INF, 0.0
    for s in range(0, x.size, block):
        xb = x[s:s + block]
        m_loc = xb.max() if xb.size else NEG_INF
        if m_loc == NEG_INF:
            continue
        l_loc = float(np.exp(xb - m_loc).sum())
        m_new = max(m, m_loc)
        l = l * math.exp(m - m_new) + l_loc * math.exp(m_loc - m_new)
        m = m_new
    return m, l


# --------------------------------------------------------------------------
# Blocked attention forward (single head)
# --------------------------------------------------------------------------

def _causal_case(q_start: int, q_end: int, k_start: int, k_end: int) -> str:
    """Classify a (Q-block, K-block) pair under the causal mask:
    'skip' if every key is after every query, 'full' if every key is at or
    before every query, else 'partial'.  ("6. FlashAttention 分块逻辑",
    section 4.1; the exact full-visibility test is k_end - 1 <= q_start.)"""
    if k_start >= q_end:
        return "skip"
    if k_end - 1 <= q_start:
        return "full"
    return "partial"


def blocked_attention(Q, K, V, Br: int, Bc: int, scale: float,
                      causal: bool = False, rescale: bool = True):
    """Tiled forward with the Q block as the outer loop and K/V blocks inner,
    running max m, running sum l and an unnormalised accumulator rescaled by
    exp(m_old - m_new), normalised once after the inner loop; the stored
    statistic is LSE = m + ln(l).  ("6. FlashAttention 分块逻辑", sections 3.1,
    3.2 and 4.2; "9.4 FlashAttention 与 FlashMLA", section 9.4.5.)

    ``rescale=False`` drops the exp(m_old - m_new) factor.  That variant is
    deliberately wrong and exists only so a test can show that the pins
    detect a missing rescale.

    Returns (O [Nq, d], LSE [Nq]).
    """
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    Nq, d = Q.shape
    Nk = K.shape[0]
    O = np.zeros((Nq, d))
    LSE = np.full(Nq, NEG_INF)
    for q_start in range(0, Nq, Br):
        q_end = min(Nq, q_start + Br)
        Qi = Q[q_start:q_end]
        rows = q_end - q_start
        acc = np.zeros((rows, d))
        m_i = np.full(rows, NEG_INF)
        l_i = np.zeros(rows)
        for k_start in range(0, Nk, Bc):
            k_end = min(Nk, k_start + Bc)
            case = _causal_case(q_start, q_end, k_start, k_end) if causal else "full"
            if case == "skip":
                continue
            S = (Qi @ K[k_start:k_end].T) * scale
            if case == "partial":
                q_pos = np.arange(q_start, q_end)[:, None]
                k_pos = np.arange(k_start, k_end)[None, :]
                S = np.where(q_pos >= k_pos, S, NEG_INF)
            m_new = np.maximum(m_i, S.max(axis=1))
            # rows with no visible key so far keep m = -inf; use 0 as the
            # reference there so that exp(-inf - 0) = 0 instead of NaN
            ref = np.where(m_new == NEG_INF, 0.0, m_new)
            alpha = np.exp(m_i - ref) if rescale else np.ones(rows)
            P = np.exp(S - ref[:, None])
            l_i = l_i * alpha + P.sum(axis=1)
            acc = acc * alpha[:, None] + P @ V[k_start:k_end]
            m_i = m_new
        seen = l_i > 0
        O[q_start:q_end][seen] = acc[seen] / l_i[seen, None]
        LSE[q_start:q_end][seen] = m_i[seen] + np.log(l_i[seen])
    return O, LSE


def blocked_attention_normalized(Q, K, V, Br: int, Bc: int, scale: float,
                                 causal: bool = False):
    """Tiled forward that keeps O normalised after every K/V block, using the
    block-local max m_ij and sum l_ij:
        m_new = max(m_i, m_ij)
        l_new = l_i exp(m_i - m_new) + l_ij exp(m_ij - m_new)
        O_i   = (l_i / l_new) exp(m_i - m_new) O_i
                + (1 / l_new) exp(m_ij - m_new) P_ij V_j
    ("9.4 FlashAttention 与 FlashMLA", section 9.4.3, forward algorithm; the
    scale is applied to the scores, as in the first page's section 3.1.)

    Returns (O [Nq, d], LSE [Nq]).
    """
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    Nq, d = Q.shape
    Nk = K.shape[0]
    O = np.zeros((Nq, d))
    LSE = np.full(Nq, NEG_INF)
    for q_start in range(0, Nq, Br):
        q_end = min(Nq, q_start + Br)
        rows = q_end - q_start
        Oi = np.zeros((rows, d))
        m_i = np.full(rows, NEG_INF)
        l_i = np.zeros(rows)
        for k_start in range(0, Nk, Bc):
            k_end = min(Nk, k_start + Bc)
            case = _causal_case(q_start, q_end, k_start, k_end) if causal else "full"
            if case == "skip":
                continue
            S = (Q[q_start:q_end] @ K[k_start:k_end].T) * scale
            if case == "partial":
                q_pos = np.arange(q_start, q_end)[:, None]
                k_pos = np.arange(k_start, k_end)[None, :]
                S = np.where(q_pos >= k_pos, S, NEG_INF)
            m_ij = S.max(axis=1)
            for r in range(rows):            # row by row: empty rows are skipped
                if m_ij[r] == NEG_INF:
                    continue
                P_r = np.exp(S[r] - m_ij[r])
                l_ij = P_r.sum()
                m_new = max(m_i[r], m_ij[r])
                l_new = l_i[r] * math.exp(m_i[r] - m_new) + l_ij * math.exp(m_ij[r] - m_new)
                Oi[r] = ((l_i[r] / l_new) * math.exp(m_i[r] - m_new) * Oi[r]
                         + (1.0 / l_new) * math.exp(m_ij[r] - m_new) * (P_r @ V[k_start:k_end]))
                m_i[r], l_i[r] = m_new, l_new
        O[q_start:q_end] = Oi
        seen = l_i > 0
        LSE[q_start:q_end][seen] = m_i[seen] + np.log(l_i[seen])
    return O, LSE


def blocked_attention_bhsd(Q, K, V, Br: int, Bc: int, scale: float,
                           causal: bool = False, normalized: bool = False):
    """Treat every (b, h) of [B, H, N, d] inputs as an independent sequence
    ("6. FlashAttention 分块逻辑", section 3.3) and run the blocked forward."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    B, H, Nq, d = Q.shape
    O = np.zeros((B, H, Nq, d))
    LSE = np.zeros((B, H, Nq))
    fn = blocked_attention_normalized if normalized else blocked_attention
    for b in range(B):
        for h in range(H):
            O[b, h], LSE[b, h] = fn(Q[b, h], K[b, h], V[b, h], Br, Bc, scale, causal)
    return O, LSE


# --------------------------------------------------------------------------
# Split-KV (decode) partials and their merge
# --------------------------------------------------------------------------

def split_bounds(Nk: int, num_splits: int):
    """Chunk c covers keys [c*chunk, min(Nk, (c+1)*chunk)) with
    chunk = ceil(Nk / num_splits); trailing chunks may be empty."""
    chunk = -(-Nk // num_splits)
    return [(min(Nk, c * chunk), min(Nk, (c + 1) * chunk)) for c in range(num_splits)]


def split_partials(q, K, V, scale: float, num_splits: int):
    """Stage one of the decode split: for each K/V chunk j independently, the
    local scores s_j = scale * q K_j^T, local max m_j, p_j = exp(s_j - m_j),
    local sum l_j and unnormalised local output o_j = p_j V_j.
    ("6. FlashAttention 分块逻辑", section 11.3, first stage.)

    Returns a list of dicts {'m', 'l', 'o'}; an empty chunk has m = -inf,
    l = 0, o = 0.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    parts = []
    for (a, b) in split_bounds(K.shape[0], num_splits):
        if b <= a:
            parts.append({"m": NEG_INF, "l": 0.0, "o": np.zeros(V.shape[1])})
            continue
        s = (K[a:b] @ q) * scale
        m = s.max()
        p = np.exp(s - m)
        parts.append({"m": float(m), "l": float(p.sum()), "o": p @ V[a:b]})
    return parts


def merge_partials(parts):
    """Stage two: fold the chunks in order with the online rule
        m_new = max(m_g, m_j)
        l_g   = l_g exp(m_g - m_new) + l_j exp(m_j - m_new)
        o_g   = o_g exp(m_g - m_new) + o_j exp(m_j - m_new)
    then o = o_g / l_g.  ("6. FlashAttention 分块逻辑", sections 11.3 and 13.2.)

    Returns (o, lse) with lse = m_g + ln(l_g).
    """
    m_g, l_g, o_g = NEG_INF, 0.0, 0.0
    for part in parts:
        if part["m"] == NEG_INF:
            continue
        m_new = max(m_g, part["m"])
        l_g = l_g * math.exp(m_g - m_new) + part["l"] * math.exp(part["m"] - m_new)
        o_g = o_g * math.exp(m_g - m_new) + part["o"] * math.exp(part["m"] - m_new)
        m_g = m_new
    return o_g / l_g, m_g + math.log(l_g)


def combine_lse(lse_c, o_tilde_c):
    """The logsumexp-weighted form of the same merge, with each chunk stored
    as (lse_c = m_c + ln l_c, o~_c = o_c / l_c):
        LSE = M + ln sum_c exp(lse_c - M),  M = max_c lse_c
        O   = sum_c exp(lse_c - LSE) o~_c
    Algebraically equal to ``merge_partials``; empty chunks (lse = -inf)
    get weight 0."""
    lse_c = np.asarray(lse_c, dtype=np.float64)
    o_tilde_c = np.asarray(o_tilde_c, dtype=np.float64)
    M = lse_c.max()
    w = np.where(lse_c == NEG_INF, 0.0, np.exp(lse_c - M))
    LSE = M + math.log(w.sum())
    weights = np.where(lse_c == NEG_INF, 0.0, np.exp(lse_c - LSE))
    return weights @ o_tilde_c, LSE


def wrong_merge(parts):
    """The faulty merge that keeps the first chunk's max forever and never
    rescales what it has accumulated ("6. FlashAttention 分块逻辑", section
    13.3).  Kept only as a negative control: it must differ from
    ``merge_partials`` whenever the chunk maxima differ."""
    m = parts[0]["m"]
    l = parts[0]["l"]
    o = np.array(parts[0]["o"], dtype=np.float64)
    for part in parts[1:]:
        l = l + part["l"] * math.exp(part["m"] - m)
        o = o + part["o"] * math.exp(part["m"] - m)
    return o / l


# --------------------------------------------------------------------------
# Paged K/V cache
# --------------------------------------------------------------------------

def paged_attention_blocked(q, k_cache, v_cache, block_table, seq_len: int, scale: float):
    """Attention of one query row over a paged cache, block by block, in the
    order the page gives ("6. FlashAttention 分块逻辑", section 12.2): for each
    logical block, look up its physical block in the table and skip it if it
    is unallocated (negative; here also >= the number of physical blocks);
    take its valid rows (all but the last block are full); form the scaled
    scores; update the running max, the running sum and the rescaled
    accumulator with the online rule; after the last block divide by the sum.

    q [d]; k_cache, v_cache [num_blocks, block_size, d] (one head);
    block_table [max_blocks].  Returns (o, lse); a row with no key gives
    (0, -inf), where the page's final division would be 0/0.
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    table = np.asarray(block_table, dtype=np.int64).reshape(-1)
    num_blocks, block_size, d = k_cache.shape
    n = max(0, min(int(seq_len), table.size * block_size))
    m, l, o = NEG_INF, 0.0, np.zeros(d)
    for lb in range(-(-n // block_size)):
        phys = int(table[lb])
        if phys < 0 or phys >= num_blocks:
            continue
        valid = min(block_size, n - lb * block_size)
        s = (k_cache[phys, :valid] @ q) * scale
        m_new = max(m, float(s.max()))
        factor = math.exp(m - m_new)
        p = np.exp(s - m_new)
        l = l * factor + float(p.sum())
        o = o * factor + p @ v_cache[phys, :valid]
        m = m_new
    if l == 0.0:
        return np.zeros(d), NEG_INF
    return o / l, m + math.log(l)


# --------------------------------------------------------------------------
# Backward by recomputation
# --------------------------------------------------------------------------

def _masked_scores(Q, K, q_start, q_end, k_start, k_end, scale, causal):
    S = (Q[q_start:q_end] @ K[k_start:k_end].T) * scale
    if causal:
        q_pos = np.arange(q_start, q_end)[:, None]
        k_pos = np.arange(k_start, k_end)[None, :]
        S = np.where(q_pos >= k_pos, S, NEG_INF)
    return S


def blocked_backward(Q, K, V, O, dO, LSE, Br: int, Bc: int, scale: float, causal: bool = False,
                     blocklocal_rowsum: bool = False):
    """The two-kernel backward ("9.4 FlashAttention 与 FlashMLA", section
    9.4.5; the block formulas of "6. FlashAttention 分块逻辑", section 7):

    * pre-pass: D_i = rowsum(dO_i * O_i);
    * dK/dV: K/V blocks outer, Q blocks inner; per pair recompute
      S = scale Q_i K_j^T (+ mask) and P = exp(S - LSE_i) from the saved
      statistic, then dV_j += P^T dO_i, dP = dO_i V_j^T,
      dS = P * (dP - D_i), dK_j += scale dS^T Q_i;
    * dQ: Q blocks outer, K/V blocks inner; the same P, dP, dS, then
      dQ_i += scale dS K_j.

    ``blocklocal_rowsum=True`` replaces D_i by the block-local sum
    rowsum(dP * P) over the current K/V block, as the first page's block
    listing writes it.  That equals D_i only when one block holds the whole
    row; the variant exists so a test can show the difference.

    Single head: Q, O, dO [Nq, d]; K, V [Nk, d]; LSE [Nq] (natural log).
    Returns (dQ, dK, dV).
    """
    Q, K, V, O, dO = (np.asarray(a, dtype=np.float64) for a in (Q, K, V, O, dO))
    LSE = np.asarray(LSE, dtype=np.float64)
    Nq, d = Q.shape
    Nk = K.shape[0]
    Dvec = (dO * O).sum(axis=1)
    dQ = np.zeros((Nq, d))
    dK = np.zeros((Nk, d))
    dV = np.zeros((Nk, d))

    def grads(q_start, q_end, k_start, k_end):
        S = _masked_scores(Q, K, q_start, q_end, k_start, k_end, scale, causal)
        P = np.exp(S - LSE[q_start:q_end, None])
        dP = dO[q_start:q_end] @ V[k_start:k_end].T
        if blocklocal_rowsum:
            Di = (dP * P).sum(axis=1, keepdims=True)
        else:
            Di = Dvec[q_start:q_end, None]
        return P, P * (dP - Di)

    for k_start in range(0, Nk, Bc):                 # dK / dV
        k_end = min(Nk, k_start + Bc)
        for q_start in range(0, Nq, Br):
            q_end = min(Nq, q_start + Br)
            if causal and _causal_case(q_start, q_end, k_start, k_end) == "skip":
                continue
            P, dS = grads(q_start, q_end, k_start, k_end)
            dV[k_start:k_end] += P.T @ dO[q_start:q_end]
            dK[k_start:k_end] += scale * (dS.T @ Q[q_start:q_end])
    for q_start in range(0, Nq, Br):                 # dQ
        q_end = min(Nq, q_start + Br)
        for k_start in range(0, Nk, Bc):
            k_end = min(Nk, k_start + Bc)
            if causal and _causal_case(q_start, q_end, k_start, k_end) == "skip":
                continue
            _, dS = grads(q_start, q_end, k_start, k_end)
            dQ[q_start:q_end] += scale * (dS @ K[k_start:k_end])
    return dQ, dK, dV
