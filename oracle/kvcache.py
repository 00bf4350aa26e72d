"""Plain float64 attention of a few new queries against a key/value cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the
product path.

What is computed, and where the pages put it
--------------------------------------------
The pages name inference next to training as what the method speeds up
("FlashAttention-2 (DE)", lead paragraph, and "Das Attention-Problem in
Transformern": Falcon-40B inference), and place the method in model serving
together with block-wise management of the key/value cache, which it is not
the same thing as ("FlashAttention" glossary, sections "Der Engpass ist der
Weg zum Speicher, nicht das Rechnen" and "Wo es verwechselt wird"; related
terms "KV Cache", "Memory-Bound", "Model Serving").  The pages give no
formula for it; the computation is the same scaled-dot-product attention as
in ``attention.py``, only with fewer queries than keys.

Per (batch, head), with Nq new queries, a cache of capacity Nk rows of which
the first L (``seqlen``, 0 <= L <= Nk) are filled:

    visible(i) = { j : j < L }                          (non-causal)
               = { j : j < L and j <= i + (L - Nq) }    (causal)

i.e. the causal mask is aligned at the bottom right: the last query sees every
filled key, the query before it one key less, and so on (the queries are the
last Nq positions of a sequence of length L).  Over visible(i):

    s_ij  = scale * q_i . k_j
    p_ij  = exp(s_ij - m_i) / sum_j' exp(s_ij' - m_i),  m_i = max_j s_ij
    O_i   = sum_j p_ij v_j
    LSE_i = m_i + ln sum_j exp(s_ij - m_i)

A query with no visible key (L = 0, or causal with i < Nq - L) has an empty
softmax; this file's convention for it is O_i = 0 and LSE_i = -inf (the
logarithm of an empty sum).  Cache rows at and past L are never read.

Two-pass softmax over the whole visible row, never online, never split over
keys.  With Nq = Nk = L this is exactly ``attention.py``'s forward (the
causal mask is then the usual top-left one).
"""

from __future__ import annotations

import numpy as np


def _visible(nq: int, seqlen: int, causal: bool) -> np.ndarray:
    """[nq, seqlen] boolean: key j visible to query i."""
    j = np.arange(seqlen)[None, :]
    if not causal:
        return np.ones((nq, seqlen), dtype=bool)
    i = np.arange(nq)[:, None]
    return j <= i + (seqlen - nq)


def kvcache_fwd_head(q, k, v, scale: float, causal: bool, seqlen: int | None = None):
    """One head. q: [Nq, d]; k, v: [Nk, d] cache; seqlen: filled rows (default Nk).

    Returns (O [Nq, d], LSE [Nq]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    nk = np.asarray(k).shape[0]
    L = nk if seqlen is None else int(seqlen)
    if not 0 <= L <= nk:
        raise ValueError("seqlen must lie in [0, Nk]")
    kk = np.asarray(k, dtype=np.float64)[:L]
    vv = np.asarray(v, dtype=np.float64)[:L]
    nq = q.shape[0]
    o = np.zeros((nq, vv.shape[1]))
    lse = np.full(nq, -np.inf)
    if L == 0:
        return o, lse
    vis = _visible(nq, L, causal)
    s = np.where(vis, scale * (q @ kk.T), -np.inf)  # s_ij over the filled keys
    rows = vis.any(axis=1)  # queries with at least one visible key
    m = s[rows].max(axis=1, keepdims=True)
    e = np.exp(s[rows] - m)
    z = e.sum(axis=1, keepdims=True)
    o[rows] = (e / z) @ vv
    lse[rows] = (m + np.log(z))[:, 0]
    return o, lse


def kvcache_fwd(q, k, v, scale: float, causal: bool, seqlens=None):
    """[B, H, Nq, d] queries against [B, H, Nk, d] caches; seqlens: [B] filled
    lengths (default: all Nk).  Returns (O [B,H,Nq,d], LSE [B,H,Nq]) float64."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    b, h, nq, _ = q.shape
    nk = k.shape[2]
    lens = [nk] * b if seqlens is None else [int(x) for x in seqlens]
    o = np.empty((b, h, nq, v.shape[-1]), dtype=np.float64)
    lse = np.empty((b, h, nq), dtype=np.float64)
    for bi in range(b):
        for hi in range(h):
            o[bi, hi], lse[bi, hi] = kvcache_fwd_head(q[bi, hi], k[bi, hi], v[bi, hi], scale, causal, lens[bi])
    return o, lse


def varlen_fwd(q, k, v, cu_q, cu_k, scale: float, causal: bool):
    """Variable-length packed batch: sequence b owns query rows
    cu_q[b] .. cu_q[b+1]-1 of q [total_q, H, d] and key/value rows
    cu_k[b] .. cu_k[b+1]-1 of k, v [total_k, H, d]; within a sequence the
    rule above applies with Nq = its query count and L = its key count
    (causal: bottom-right aligned).  Returns (O [total_q, H, d],
    LSE [H, total_q]) in float64; rows of no sequence stay 0 / -inf."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    tq, h, d = q.shape
    o = np.zeros((tq, h, v.shape[2]))
    lse = np.full((h, tq), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 <= q0:
            continue
        for hi in range(h):
            ob, lb = kvcache_fwd_head(q[q0:q1, hi], k[k0:k1, hi], v[k0:k1, hi], scale, causal)
            o[q0:q1, hi] = ob
            lse[hi, q0:q1] = lb
    return o, lse


def varlen_bwd_causal(q, k, v, do, cu, scale: float):
    """Gradient of causal self-attention over a packed variable-length batch:
    sequence b owns rows cu[b] .. cu[b+1]-1 of q, k, v, do (each [total, H, d]),
    with as many queries as keys.  Per sequence and head this is the pinned
    ``attention_bwd_head`` of ``attention.py`` (softmax Jacobian, causal).
    Returns (dQ, dK, dV) [total, H, d] float64; rows of no sequence stay 0."""
    from .attention import attention_bwd_head
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    tot, h, d = q.shape
    dq, dk, dv = (np.zeros((tot, h, d)) for _ in range(3))
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 <= s0:
            continue
        for hi in range(h):
            g = attention_bwd_head(q[s0:s1, hi], k[s0:s1, hi], v[s0:s1, hi], do[s0:s1, hi], scale, True)
            dq[s0:s1, hi], dk[s0:s1, hi], dv[s0:s1, hi] = g
    return dq, dk, dv


def kvcache_bwd_head(q, k, v, do, scale: float, causal: bool, seqlen: int | None = None):
    """Gradient of ``kvcache_fwd_head``'s O with respect to q, k, v for the
    upstream gradient do ([Nq, d]): the chain rule through the softmax over
    each query's visible keys (the bottom-right mask above), written out as
    the softmax Jacobian, in float64:

        dV_j  = sum_i p_ij dO_i
        dP_ij = dO_i . v_j
        dS_ij = p_ij (dP_ij - sum_j' p_ij' dP_ij')
        dQ_i  = scale sum_j dS_ij k_j
        dK_j  = scale sum_i dS_ij q_i

    A query with no visible key has the constant output 0: it adds nothing
    and its dQ is 0.  Cache rows at and past the filled length get zero
    gradients.  Returns (dQ [Nq, d], dK [Nk, d], dV [Nk, d])."""
    q = np.asarray(q, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    nk = np.asarray(k).shape[0]
    L = nk if seqlen is None else int(seqlen)
    kk = np.asarray(k, dtype=np.float64)[:L]
    vv = np.asarray(v, dtype=np.float64)[:L]
    nq, d = q.shape
    dq = np.zeros((nq, d))
    dk = np.zeros((nk, kk.shape[1] if L else d))
    dv = np.zeros((nk, vv.shape[1] if L else d))
    if L == 0:
        return dq, dk, dv
    vis = _visible(nq, L, causal)
    s = np.where(vis, scale * (q @ kk.T), -np.inf)
    rows = vis.any(axis=1)
    p = np.zeros((nq, L))
    m = s[rows].max(axis=1, keepdims=True)
    e = np.exp(s[rows] - m)
    p[rows] = e / e.sum(axis=1, keepdims=True)  # 0 at masked keys and in empty rows
    dv[:L] = p.T @ do
    dp = do @ vv.T
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    dq[:] = scale * (ds @ kk)
    dk[:L] = scale * (ds.T @ q)
    return dq, dk, dv


def varlen_bwd(q, k, v, do, cu_q, cu_k, scale: float, causal: bool):
    """Gradient of ``varlen_fwd``'s O for the upstream gradient do
    [total_q, H, d]: per sequence and head ``kvcache_bwd_head`` with that
    sequence's query and key rows (any counts; causal bottom-right aligned).
    Returns (dQ [total_q, H, d], dK, dV [total_k, H, d]) in float64; rows of
    no sequence stay 0."""
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    tq, h, d = q.shape
    tk = k.shape[0]
    dq, dk, dv = np.zeros((tq, h, d)), np.zeros((tk, h, d)), np.zeros((tk, h, v.shape[2]))
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 <= q0 and k1 <= k0:
            continue
        for hi in range(h):
            g = kvcache_bwd_head(q[q0:q1, hi], k[k0:k1, hi], v[k0:k1, hi], do[q0:q1, hi], scale, causal)
            dq[q0:q1, hi], dk[k0:k1, hi], dv[k0:k1, hi] = g
    return dq, dk, dv
