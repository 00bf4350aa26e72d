"""Plain float64 attention: the definition the tiled GPU method must reproduce.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the
product path.

What is computed, and where the pages fix it
--------------------------------------------
The pages ("FlashAttention-2 (DE)", lead paragraphs; "FlashAttention" glossary,
section "Wo es verwechselt wird"; "FlashAttention" lexicon, "Methodische
Grundlagen", paragraph "Exaktheit") state that the method computes exactly the
usual attention, only in a different order, identical up to ordinary rounding.
The pages never write the formula out, so this file writes out the plain
definition of scaled-dot-product attention, per (batch, head):

    s_ij  = scale * sum_k q_ik k_jk              for keys j allowed for row i
    m_i   = max_j s_ij
    p_ij  = exp(s_ij - m_i) / sum_j' exp(s_ij' - m_i)
    O_i   = sum_j p_ij v_j
    LSE_i = m_i + ln sum_j exp(s_ij - m_i)       (natural log, scaled scores)

Allowed keys: all j for non-causal attention; j <= i (lower triangle, top-left
aligned, equal query and key lengths) for causal attention.

This is the *standard* two-pass softmax: the full row of scores is formed
before normalising.  It never uses the running (online) normalisation that the
lexicon page describes under "Fortlaufende Normierung", and it never tiles over
keys, so it shares no arithmetic structure with the tiled kernels it checks.

The backward pass follows the lexicon's "Neuberechnung statt Speicherung"
(the score matrix is rebuilt, here simply recomputed from Q and K); its
formulas are not on the pages and come from the chain rule through the softmax
Jacobian, given the upstream gradient dO:

    dV_j  = sum_i p_ij dO_i
    dP_ij = dO_i . v_j
    dS_ij = p_ij (dP_ij - sum_k p_ik dP_ik)
    dQ_i  = scale * sum_j dS_ij k_j
    dK_j  = scale * sum_i dS_ij q_i

Arrays are float64 throughout.  Inputs of any float dtype are converted to
float64 first (bf16/fp16/fp32 values are exact in float64).  Work is chunked by
head and by blocks of at most ``ROW_CHUNK`` query rows, so that long sequences
fit in host memory; for causal attention a chunk only forms the key prefix it
can see.  Chunking over rows does not change any row's arithmetic.
"""

from __future__ import annotations

import numpy as np

ROW_CHUNK = 1024


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _row_probs(q_rows: np.ndarray, k: np.ndarray, rows: np.ndarray, scale: float, causal: bool):
    """Scores, probabilities and LSE for the given query rows of one head.

    q_rows: [r, d] float64 query rows; rows: their row indices i; k: [Nk, d].
    Returns (p [r, Nk'], lse [r], nk') where only the first nk' keys are formed
    (for causal attention keys beyond the last row of the chunk are never
    allowed, so they are not formed).
    """
    nk = k.shape[0]
    if causal:
        nk = min(nk, int(rows.max()) + 1)
    s = scale * (q_rows @ k[:nk].T)  # s_ij = scale * q_i . k_j
    if causal:
        allowed = np.arange(nk)[None, :] <= rows[:, None]
        s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)  # m_i = max over allowed keys
    e = np.exp(s - m)  # exp(-inf) = 0 for keys that are not allowed
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    lse = (m + np.log(z))[:, 0]
    return p, lse, nk


def attention_fwd_head(q, k, v, scale: float, causal: bool, rows=None):
    """Forward of one head. q: [N, d], k, v: [N, d].

    Returns (O [r, d], LSE [r]) for the requested ``rows`` (all rows when None),
    in float64.  ``rows`` lets a test check sampled rows of a very long
    sequence one by one without forming the whole head.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    n = q.shape[0]
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.empty(rows.shape[0], dtype=np.float64)
    for c0 in range(0, rows.shape[0], ROW_CHUNK):
        r = rows[c0:c0 + ROW_CHUNK]
        p, l, nk = _row_probs(q[r], k, r, scale, causal)
        o[c0:c0 + r.shape[0]] = p @ v[:nk]  # O_i = sum_j p_ij v_j
        lse[c0:c0 + r.shape[0]] = l
    return o, lse


def attention_fwd(q, k, v, scale: float, causal: bool):
    """Forward over [B, H, N, d] inputs. Returns (O [B,H,N,d], LSE [B,H,N]) float64."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    b, h, n, _ = q.shape
    o = np.empty((b, h, n, v.shape[-1]), dtype=np.float64)
    lse = np.empty((b, h, n), dtype=np.float64)
    for bi in range(b):
        for hi in range(h):
            o[bi, hi], lse[bi, hi] = attention_fwd_head(q[bi, hi], k[bi, hi], v[bi, hi], scale, causal)
    return o, lse


def attention_bwd_head(q, k, v, do, scale: float, causal: bool):
    """Gradient of one head through the softmax Jacobian. All inputs [N, d].

    Returns (dQ, dK, dV), each [N, d] float64.  P is rebuilt from Q and K
    chunk by chunk (nothing from the forward is reused).
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    n = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for c0 in range(0, n, ROW_CHUNK):
        r = np.arange(c0, min(n, c0 + ROW_CHUNK))
        p, _, nk = _row_probs(q[r], k, r, scale, causal)
        g = do[r]
        dv[:nk] += p.T @ g  # dV_j = sum_i p_ij dO_i
        dp = g @ v[:nk].T  # dP_ij = dO_i . v_j
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))  # softmax Jacobian
        dq[r] = scale * (ds @ k[:nk])  # dQ_i = scale sum_j dS_ij k_j
        dk[:nk] += scale * (ds.T @ q[r])  # dK_j = scale sum_i dS_ij q_i
    return dq, dk, dv


def attention_bwd(q, k, v, do, scale: float, causal: bool):
    """Gradient over [B, H, N, d] inputs. Returns (dQ, dK, dV) float64."""
    b, h, n, d = np.asarray(q).shape
    dq = np.empty((b, h, n, d), dtype=np.float64)
    dk = np.empty((b, h, n, d), dtype=np.float64)
    dv = np.empty((b, h, n, d), dtype=np.float64)
    for bi in range(b):
        for hi in range(h):
            dq[bi, hi], dk[bi, hi], dv[bi, hi] = attention_bwd_head(
                q[bi, hi], k[bi, hi], v[bi, hi], do[bi, hi], scale, causal)
    return dq, dk, dv
