"""Pins for the float64 key/value-cache oracle (``oracle/kvcache.py``), all on
the CPU, each checked against something other than the function itself: the
40-digit decimal brute force, the already pinned square-attention oracle
(``attention.py``) on the same sequence, and identities of exact attention.
``test_kvcache_mutations_are_caught`` plants plausible mistakes in a copy of
the source and checks that the battery catches each one.
"""

import math
import types

import numpy as np
import pytest

from oracle import attention_fwd_head, brute_kvcache_decimal, kvcache_fwd, kvcache_fwd_head, varlen_fwd
from oracle import kvcache as okv


def rnd(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def _dec(o, lse):
    return (np.array([[float(x) for x in r] for r in o]).reshape(len(o), -1),
            np.array([float(x) for x in lse]))


CASES = [(1, 1, 1), (1, 5, 5), (1, 6, 3), (2, 4, 4), (3, 7, 5), (5, 8, 8), (4, 6, 2), (3, 3, 0), (2, 5, 1)]


@pytest.mark.parametrize("nq,nk,L", CASES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.7, -0.55])
def test_kvcache_matches_decimal_brute_force(nq, nk, L, causal, scale):
    rng = np.random.default_rng(500 + 11 * nq + 3 * nk + L)
    d = 3
    q, k, v = rnd(rng, nq, d, s=1.5), rnd(rng, nk, d, s=1.5), rnd(rng, nk, d)
    o, lse = kvcache_fwd_head(q, k, v, scale, causal, L)
    ob, lb = _dec(*brute_kvcache_decimal(q, k, v, scale, causal, L))
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    assert np.max(np.abs(o - ob), initial=0.0) <= 1e-12
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0.0) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_square_case_is_the_ordinary_forward(causal):
    rng = np.random.default_rng(7)
    n, d = 37, 8
    q, k, v = rnd(rng, n, d), rnd(rng, n, d), rnd(rng, n, d)
    o, lse = kvcache_fwd_head(q, k, v, 1 / math.sqrt(d), causal)
    o2, lse2 = attention_fwd_head(q, k, v, 1 / math.sqrt(d), causal)
    assert np.max(np.abs(o - o2)) <= 1e-13 and np.max(np.abs(lse - lse2)) <= 1e-13


@pytest.mark.parametrize("nq,L", [(1, 40), (5, 40), (40, 40), (7, 9)])
def test_causal_queries_are_the_last_rows_of_the_full_sequence(nq, L):
    """Bottom-right alignment: the Nq queries are positions L-Nq .. L-1 of a
    sequence of length L, so they equal those rows of ordinary causal attention."""
    rng = np.random.default_rng(8 + nq)
    d = 6
    k, v = rnd(rng, L + 5, d), rnd(rng, L + 5, d)
    qfull = rnd(rng, L, d)
    o, lse = kvcache_fwd_head(qfull[L - nq:], k, v, 0.4, True, L)
    of, lf = attention_fwd_head(qfull, k[:L], v[:L], 0.4, True)
    assert np.max(np.abs(o - of[L - nq:])) <= 1e-13
    assert np.max(np.abs(lse - lf[L - nq:])) <= 1e-13


def test_single_query_sees_every_filled_key():
    rng = np.random.default_rng(9)
    q, k, v = rnd(rng, 1, 4), rnd(rng, 30, 4), rnd(rng, 30, 4)
    for L in (1, 17, 30):
        a = kvcache_fwd_head(q, k, v, 0.5, True, L)
        b = kvcache_fwd_head(q, k, v, 0.5, False, L)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rows_past_the_filled_length_are_never_read():
    rng = np.random.default_rng(10)
    q, k, v = rnd(rng, 3, 4), rnd(rng, 20, 4), rnd(rng, 20, 4)
    k2, v2 = k.copy(), v.copy()
    k2[12:] = np.nan
    v2[12:] = np.inf
    for causal in (False, True):
        a = kvcache_fwd_head(q, k, v, 0.5, causal, 12)
        b = kvcache_fwd_head(q, k2, v2, 0.5, causal, 12)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_empty_rows_convention():
    rng = np.random.default_rng(11)
    q, k, v = rnd(rng, 4, 3), rnd(rng, 6, 3), rnd(rng, 6, 3)
    o, lse = kvcache_fwd_head(q, k, v, 0.5, False, 0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # causal with L = 2 < Nq = 4: queries 0 and 1 see nothing, query 2 sees key 0
    o, lse = kvcache_fwd_head(q, k, v, 0.5, True, 2)
    assert np.all(o[:2] == 0) and np.all(np.isneginf(lse[:2]))
    assert np.max(np.abs(o[2] - v[0])) <= 1e-15
    assert abs(lse[2] - 0.5 * q[2] @ k[0]) <= 1e-14


def test_zero_queries_give_mean_of_visible_values():
    rng = np.random.default_rng(12)
    k, v = rnd(rng, 10, 3), rnd(rng, 10, 3)
    q = np.zeros((3, 3))
    o, lse = kvcache_fwd_head(q, k, v, 0.5, True, 8)
    for i in range(3):
        n_vis = 8 - 3 + i + 1
        assert np.max(np.abs(o[i] - v[:n_vis].mean(axis=0))) <= 1e-14
        assert abs(lse[i] - math.log(n_vis)) <= 1e-14


def test_split_keys_merge_to_the_whole():
    """The identity a split-key computation relies on: partial results over
    disjoint key ranges combine through their log-sum-exps,
    LSE = ln sum_s e^{LSE_s},  O = sum_s e^{LSE_s - LSE} O_s."""
    rng = np.random.default_rng(13)
    q, k, v = rnd(rng, 3, 5, s=2), rnd(rng, 50, 5, s=2), rnd(rng, 50, 5)
    o, lse = kvcache_fwd_head(q, k, v, 0.6, False, 50)
    parts = [kvcache_fwd_head(q, k[a:b], v[a:b], 0.6, False) for a, b in ((0, 7), (7, 30), (30, 50))]
    ls = np.stack([p[1] for p in parts])
    top = ls.max(axis=0)
    lse_m = top + np.log(np.exp(ls - top).sum(axis=0))
    o_m = sum(np.exp(p[1] - lse_m)[:, None] * p[0] for p in parts)
    assert np.max(np.abs(lse_m - lse)) <= 1e-13 and np.max(np.abs(o_m - o)) <= 1e-13


def test_batched_with_lengths_matches_per_head():
    rng = np.random.default_rng(14)
    q, k, v = rnd(rng, 3, 2, 4, 5), rnd(rng, 3, 2, 9, 5), rnd(rng, 3, 2, 9, 5)
    lens = [9, 0, 4]
    o, lse = kvcache_fwd(q, k, v, 0.3, True, lens)
    for b in range(3):
        for h in range(2):
            oo, ll = kvcache_fwd_head(q[b, h], k[b, h], v[b, h], 0.3, True, lens[b])
            assert np.array_equal(o[b, h], oo) and np.array_equal(lse[b, h], ll)


# ---------------------------------------------------------------- mutation check

def _kv_pins_pass(mod) -> bool:
    rng = np.random.default_rng(41)
    try:
        for causal in (False, True):
            for nq, nk, L in ((3, 7, 5), (4, 6, 2), (1, 4, 4), (2, 3, 0)):
                q, k, v = rnd(rng, nq, 3, s=1.5), rnd(rng, nk, 3, s=1.5), rnd(rng, nk, 3)
                k[L:] = np.nan
                v[L:] = np.nan
                o, lse = mod.kvcache_fwd_head(q, k, v, 0.7, causal, L)
                ob, lb = _dec(*brute_kvcache_decimal(q, k, v, 0.7, causal, L))
                if not np.array_equal(np.isneginf(lse), np.isneginf(lb)):
                    return False
                fin = np.isfinite(lb)
                if not np.max(np.abs(o - ob), initial=0.0) <= 1e-12:
                    return False
                if not np.max(np.abs(lse[fin] - lb[fin]), initial=0.0) <= 1e-12:
                    return False
        return True
    except Exception:
        return False


KV_MUTATIONS = [
    ("mask aligned top-left", "return j <= i + (seqlen - nq)", "return j <= i"),
    ("mask off by one", "return j <= i + (seqlen - nq)", "return j < i + (seqlen - nq)"),
    ("mask offset sign", "return j <= i + (seqlen - nq)", "return j <= i - (seqlen - nq)"),
    ("filled length ignored", "kk = np.asarray(k, dtype=np.float64)[:L]", "kk = np.asarray(k, dtype=np.float64)[:nk]"),
    ("scale dropped", "s = np.where(vis, scale * (q @ kk.T), -np.inf)", "s = np.where(vis, (q @ kk.T), -np.inf)"),
    ("not normalised", "o[rows] = (e / z) @ vv", "o[rows] = e @ vv"),
    ("lse drops the max", "lse[rows] = (m + np.log(z))[:, 0]", "lse[rows] = (np.log(z))[:, 0]"),
    ("empty rows get lse 0", "lse = np.full(nq, -np.inf)", "lse = np.zeros(nq)"),
]


def test_unmutated_kvcache_oracle_passes_battery():
    assert _kv_pins_pass(okv)


@pytest.mark.parametrize("label,old,new", KV_MUTATIONS, ids=[m[0] for m in KV_MUTATIONS])
def test_kvcache_mutations_are_caught(label, old, new):
    src = open(okv.__file__).read()
    assert old in src, f"mutation anchor not found: {label}"
    mod = types.ModuleType("kv_mutant")
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    assert not _kv_pins_pass(mod), f"pins did not catch mutation: {label}"


# ---------------------------------------------------------------- variable-length packed batches

def _pack(x, lens):
    """[B, H, n, d] (first lens[b] rows of each b) -> packed [sum lens, H, d]."""
    return np.concatenate([x[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)], axis=0)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_is_the_batched_call(causal):
    rng = np.random.default_rng(60)
    B, H, nq, nk, d = 3, 2, 5, 9, 4
    q, k, v = rnd(rng, B, H, nq, d), rnd(rng, B, H, nk, d), rnd(rng, B, H, nk, d)
    o, lse = kvcache_fwd(q, k, v, 0.5, causal)
    cu_q, cu_k = np.arange(B + 1) * nq, np.arange(B + 1) * nk
    ov, lv = varlen_fwd(_pack(q, [nq] * B), _pack(k, [nk] * B), _pack(v, [nk] * B), cu_q, cu_k, 0.5, causal)
    assert np.array_equal(ov, _pack(o, [nq] * B))
    assert np.array_equal(lv, np.concatenate([lse[b] for b in range(B)], axis=1))


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_matches_decimal_brute_force(causal):
    rng = np.random.default_rng(61)
    lq, lk = [2, 0, 3, 1], [3, 2, 2, 0]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    H, d = 2, 3
    q, k, v = rnd(rng, cu_q[-1], H, d, s=1.5), rnd(rng, cu_k[-1], H, d, s=1.5), rnd(rng, cu_k[-1], H, d)
    o, lse = varlen_fwd(q, k, v, cu_q, cu_k, 0.7, causal)
    for b in range(len(lq)):
        for h in range(H):
            qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
            if lq[b] == 0:
                continue
            if lk[b] == 0:  # no keys: the empty-row convention
                assert np.all(o[qs, h] == 0) and np.all(np.isneginf(lse[h, qs]))
                continue
            ob, lb = _dec(*brute_kvcache_decimal(q[qs, h], k[ks, h], v[ks, h], 0.7, causal, lk[b]))
            assert np.max(np.abs(o[qs, h] - ob)) <= 1e-12
            fin = np.isfinite(lb)
            assert np.array_equal(np.isneginf(lse[h, qs]), np.isneginf(lb))
            assert np.max(np.abs(lse[h, qs][fin] - lb[fin]), initial=0.0) <= 1e-12


def test_varlen_sequences_are_independent():
    """Changing one sequence's keys changes only that sequence's outputs."""
    rng = np.random.default_rng(62)
    lq, lk = [3, 4], [5, 6]
    cu_q, cu_k = np.array([0, 3, 7]), np.array([0, 5, 11])
    q, k, v = rnd(rng, 7, 2, 4), rnd(rng, 11, 2, 4), rnd(rng, 11, 2, 4)
    o1, l1 = varlen_fwd(q, k, v, cu_q, cu_k, 0.5, True)
    k2 = k.copy()
    k2[5:] += rnd(rng, 6, 2, 4)  # (a common shift of all keys would change nothing)
    o2, l2 = varlen_fwd(q, k2, v, cu_q, cu_k, 0.5, True)
    assert np.array_equal(o1[:3], o2[:3]) and np.array_equal(l1[:, :3], l2[:, :3])
    assert not np.allclose(o1[3:], o2[3:])


def test_varlen_backward_equal_lengths_is_the_batched_gradient():
    from oracle import attention_bwd, varlen_bwd_causal
    rng = np.random.default_rng(63)
    B, H, n, d = 3, 2, 6, 4
    q, k, v, do = (rnd(rng, B, H, n, d) for _ in range(4))
    g = attention_bwd(q, k, v, do, 0.5, True)
    cu = np.arange(B + 1) * n
    gv = varlen_bwd_causal(*(_pack(x, [n] * B) for x in (q, k, v, do)), cu, 0.5)
    for a, b in zip(gv, g):
        assert np.array_equal(a, _pack(b, [n] * B))


def test_varlen_backward_matches_finite_differences_of_the_forward():
    """Central differences of sum(O * dO) through the varlen forward oracle,
    ragged lengths (including an empty sequence)."""
    from oracle import varlen_bwd_causal
    rng = np.random.default_rng(64)
    lens = [3, 0, 2, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    tot, H, d, sc = int(cu[-1]), 2, 3, 0.6
    q, k, v, do = (rnd(rng, tot, H, d) for _ in range(4))
    dq, dk, dv = varlen_bwd_causal(q, k, v, do, cu, sc)
    f = lambda q_, k_, v_: float(np.sum(varlen_fwd(q_, k_, v_, cu, cu, sc, True)[0] * do))
    eps = 1e-6
    for which, g in ((0, dq), (1, dk), (2, dv)):
        for idx in np.ndindex(tot, H, d):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            fp = f(*args)
            args[which][idx] -= 2 * eps
            fm = f(*args)
            assert abs((fp - fm) / (2 * eps) - g[idx]) <= 1e-7



# ---------------------------------------------------------------- gradient with unequal counts

def _kv_grad_fd_ok(mod, nq, nk, L, causal, seed, tol=1e-7):
    """Central differences of sum(O * dO) through kvcache_fwd_head, every
    input element, against mod.kvcache_bwd_head."""
    rng = np.random.default_rng(seed)
    q, k, v, do = rnd(rng, nq, 3, s=1.2), rnd(rng, nk, 3, s=1.2), rnd(rng, nk, 3), rnd(rng, nq, 3)
    sc = 0.7
    dq, dk, dv = mod.kvcache_bwd_head(q, k, v, do, sc, causal, L)
    f = lambda q_, k_, v_: float(np.sum(okv.kvcache_fwd_head(q_, k_, v_, sc, causal, L)[0] * do))
    eps = 1e-6
    for which, g in ((0, dq), (1, dk), (2, dv)):
        base = (q, k, v)[which]
        for idx in np.ndindex(*base.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            fp = f(*args)
            args[which][idx] -= 2 * eps
            fm = f(*args)
            if not abs((fp - fm) / (2 * eps) - g[idx]) <= tol:
                return False
    return True


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk,L", [(3, 7, 5), (5, 4, 4), (6, 6, 2), (1, 4, 4), (4, 4, 4), (2, 3, 0)])
def test_kvcache_backward_matches_finite_differences(nq, nk, L, causal):
    """Fewer and more queries than keys, a partly filled cache, empty rows
    (causal with nq > L), the square case and an empty cache."""
    assert _kv_grad_fd_ok(okv, nq, nk, L, causal, seed=70 + nq + 3 * L)


@pytest.mark.parametrize("causal", [False, True])
def test_kvcache_backward_square_case_is_the_ordinary_gradient(causal):
    from oracle import attention_bwd_head
    rng = np.random.default_rng(71)
    q, k, v, do = (rnd(rng, 9, 4) for _ in range(4))
    for a, b in zip(okv.kvcache_bwd_head(q, k, v, do, 0.4, causal), attention_bwd_head(q, k, v, do, 0.4, causal)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_kvcache_backward_invariants():
    """Rows of P sum to 1 over visible keys: sum_j dV_j = sum of dO over rows
    with a visible key; a common shift of all keys leaves O unchanged, so
    sum_j dK_j = 0; unfilled cache rows get zero gradients."""
    rng = np.random.default_rng(72)
    nq, nk, L = 6, 8, 5
    q, k, v, do = rnd(rng, nq, 3), rnd(rng, nk, 3), rnd(rng, nk, 3), rnd(rng, nq, 3)
    dq, dk, dv = okv.kvcache_bwd_head(q, k, v, do, 0.8, True, L)
    seen = (np.arange(nq)[:, None] + (L - nq) >= 0).ravel()  # rows with a visible key
    np.testing.assert_allclose(dv.sum(axis=0), do[seen].sum(axis=0), atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    assert not dk[L:].any() and not dv[L:].any()
    assert not dq[~seen].any()


def test_varlen_backward_general_is_per_sequence_and_reduces_to_the_causal_one():
    from oracle import varlen_bwd, varlen_bwd_causal
    rng = np.random.default_rng(73)
    lq, lk = [3, 0, 5, 2], [4, 2, 3, 2]
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    H, d = 2, 3
    q, do = rnd(rng, int(cq[-1]), H, d), rnd(rng, int(cq[-1]), H, d)
    k, v = rnd(rng, int(ck[-1]), H, d), rnd(rng, int(ck[-1]), H, d)
    for causal in (False, True):
        dq, dk, dv = varlen_bwd(q, k, v, do, cq, ck, 0.5, causal)
        for b in range(4):
            for h in range(H):
                g = okv.kvcache_bwd_head(q[cq[b]:cq[b + 1], h], k[ck[b]:ck[b + 1], h], v[ck[b]:ck[b + 1], h],
                                         do[cq[b]:cq[b + 1], h], 0.5, causal)
                assert np.array_equal(dq[cq[b]:cq[b + 1], h], g[0])
                assert np.array_equal(dk[ck[b]:ck[b + 1], h], g[1])
                assert np.array_equal(dv[ck[b]:ck[b + 1], h], g[2])
    # equal counts, causal: the self-attention gradient
    lens = [4, 1, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = [rnd(rng, int(cu[-1]), H, d) for _ in range(4)]
    for a, b in zip(varlen_bwd(*x, cu, cu, 0.5, True), varlen_bwd_causal(*x, cu, 0.5)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


KV_BWD_MUTATIONS = [
    ("dV from dO without P", "dv[:L] = p.T @ do", "dv[:L] = np.ones_like(p).T @ do"),
    ("Jacobian sign", "ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))",
     "ds = p * (dp + np.sum(p * dp, axis=1, keepdims=True))"),
    ("Jacobian term missing", "ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))", "ds = p * dp"),
    ("dQ scale missing", "dq[:] = scale * (ds @ kk)", "dq[:] = (ds @ kk)"),
    ("dK from the wrong operand", "dk[:L] = scale * (ds.T @ q)", "dk[:L] = scale * (ds.T @ do)"),
    ("backward mask top-left", "s = np.where(vis, scale * (q @ kk.T), -np.inf)\n    rows = vis.any(axis=1)\n    p = ",
     "s = np.where(_visible(nq, L, False) if False else (np.arange(L)[None, :] <= np.arange(nq)[:, None]) "
     "if causal else vis, scale * (q @ kk.T), -np.inf)\n    rows = vis.any(axis=1)\n    p = "),
]


@pytest.mark.parametrize("label,old,new", KV_BWD_MUTATIONS, ids=[m[0] for m in KV_BWD_MUTATIONS])
def test_kvcache_backward_mutations_are_caught(label, old, new):
    src = open(okv.__file__).read()
    assert old in src, f"mutation anchor not found: {label}"
    mod = types.ModuleType("kv_bwd_mutant")
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    ok = all(_kv_grad_fd_ok(mod, nq, nk, L, causal, seed=80 + nq)
             for causal in (False, True) for nq, nk, L in ((3, 7, 5), (5, 4, 4)))
    assert not ok, f"finite differences did not catch mutation: {label}"
