"""Brute-force attention forward in 40-digit decimal arithmetic, for tiny shapes.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

It pins ``attention.py`` from outside float64: plain Python loops over
``decimal.Decimal`` with ``exp``/``ln`` taken from the standard library at a
working precision of 40 significant digits.  It follows the definition of
scaled-dot-product attention written in ``attention.py``'s header (the pages
call the method an exact reordering of that computation: "FlashAttention"
lexicon, "Methodische Grundlagen", paragraph "Exaktheit"), but is written
independently: no max-subtraction (not needed at 40 digits), no numpy, no
chunking.

Inputs are nested Python sequences (or arrays) of shape [N][d]; floats are
converted exactly (``Decimal(float)`` is exact).
"""

from __future__ import annotations

from decimal import Decimal, localcontext


def brute_fwd_decimal(q, k, v, scale, causal: bool, prec: int = 40):
    """Return (O, LSE) for one head as nested lists of Decimal.

    O[i][c] = sum_j w_ij v[j][c] with w_ij = e^{scale q_i.k_j} / sum_j' e^{scale q_i.k_j'}
    LSE[i]  = ln sum_j e^{scale q_i.k_j}
    where j (and j') range over all keys, or over j <= i when ``causal``.
    """
    with localcontext() as ctx:
        ctx.prec = prec
        sc = Decimal(float(scale)) if not isinstance(scale, Decimal) else scale
        n = len(q)
        d = len(q[0])
        dv = len(v[0])
        qd = [[Decimal(float(x)) for x in row] for row in q]
        kd = [[Decimal(float(x)) for x in row] for row in k]
        vd = [[Decimal(float(x)) for x in row] for row in v]
        out, lse = [], []
        for i in range(n):
            keys = range(i + 1) if causal else range(len(k))
            weights = []
            for j in keys:
                dot = sum((qd[i][c] * kd[j][c] for c in range(d)), Decimal(0))
                weights.append((j, (sc * dot).exp()))
            z = sum((w for _, w in weights), Decimal(0))
            row = []
            for c in range(dv):
                acc = sum((w * vd[j][c] for j, w in weights), Decimal(0))
                row.append(acc / z)
            out.append(row)
            lse.append(z.ln())
        return out, lse


def brute_kvcache_decimal(q, k, v, scale, causal: bool, seqlen: int, prec: int = 40):
    """Nq queries against the first ``seqlen`` rows of a key/value cache, one
    head, in 40-digit decimal: (O, LSE) as nested lists of Decimal.

    Query i (0-based, of Nq) sees key j iff j < seqlen and, when ``causal``,
    j - i <= seqlen - Nq (bottom-right aligned mask).  A query that sees no
    key gets O = 0 and LSE = -Infinity.
    """
    with localcontext() as ctx:
        ctx.prec = prec
        sc = Decimal(float(scale))
        nq, d, dv = len(q), len(q[0]), len(v[0])
        out, lse = [], []
        for i in range(nq):
            keys = [j for j in range(seqlen) if not causal or j - i <= seqlen - nq]
            if not keys:
                out.append([Decimal(0)] * dv)
                lse.append(Decimal("-Infinity"))
                continue
            weights = []
            for j in keys:
                dot = sum((Decimal(float(q[i][c])) * Decimal(float(k[j][c])) for c in range(d)), Decimal(0))
                weights.append((j, (sc * dot).exp()))
            z = sum((w for _, w in weights), Decimal(0))
            out.append([sum((w * Decimal(float(v[j][c])) for j, w in weights), Decimal(0)) / z
                        for c in range(dv)])
            lse.append(z.ln())
        return out, lse
