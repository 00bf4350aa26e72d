"""Pins for the float64 oracle, checked against things other than itself.

Every check here runs on the CPU.  The pages print no worked example and no
output values, so the pins are: a 40-digit decimal brute force, closed forms,
invariants of exact attention, central finite differences of the forward, and
an independent library implementation (torch float64 autograd) used as a cross
check only.  ``test_mutations_are_caught`` plants plausible mistakes in a copy
of the oracle's source and checks that these pins catch each one.
"""

import json
import math
import os
import types

import numpy as np
import pytest

import oracle
from oracle import attention as oatt
from oracle import attention_bwd_head, attention_fwd, attention_fwd_head, brute_fwd_decimal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SHAPES_TINY = [(1, 1), (2, 1), (3, 2), (5, 4), (8, 2), (17, 4)]


def rnd(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("n,d", SHAPES_TINY)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_forward_matches_decimal_brute_force(n, d, causal, sign):
    # sign -1: softmax(scale QK^T) for a negative scale, defined like any other
    # (the weights favour the keys of smallest q.k)
    rng = np.random.default_rng(100 + 7 * n + d)
    q, k, v = rnd(rng, n, d, s=1.5), rnd(rng, n, d, s=1.5), rnd(rng, n, d)
    scale = sign / math.sqrt(d)
    o, lse = attention_fwd_head(q, k, v, scale, causal)
    ob, lb = brute_fwd_decimal(q, k, v, scale, causal)
    ob = np.array([[float(x) for x in r] for r in ob])
    lb = np.array([float(x) for x in lb])
    assert np.max(np.abs(o - ob)) <= 1e-12
    assert np.max(np.abs(lse - lb)) <= 1e-12


def test_forward_matches_golden_fixture():
    """Values written by tests/golden/make_golden.py from the decimal brute force."""
    with open(os.path.join(GOLDEN, "brute_small.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        q, k, v = (np.array(case[x]) for x in ("q", "k", "v"))
        o, lse = attention_fwd_head(q, k, v, case["scale"], case["causal"])
        assert np.max(np.abs(o - np.array(case["o"]))) <= 1e-12
        assert np.max(np.abs(lse - np.array(case["lse"]))) <= 1e-12


# ---------------------------------------------------------------- closed forms

def test_two_keys_logistic_closed_form():
    """N = 2, d = 1, non-causal: the weight of key 0 is the logistic function
    of the score difference; LSE = s0 + ln(1 + e^{s1 - s0})."""
    q = np.array([[0.7], [-1.3]])
    k = np.array([[1.1], [-0.4]])
    v = np.array([[2.0], [-3.0]])
    scale = 0.9
    o, lse = attention_fwd_head(q, k, v, scale, False)
    for i in range(2):
        s0, s1 = scale * q[i, 0] * k[0, 0], scale * q[i, 0] * k[1, 0]
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        assert abs(o[i, 0] - (w0 * 2.0 + (1 - w0) * -3.0)) <= 1e-14
        assert abs(lse[i] - (s0 + math.log1p(math.exp(s1 - s0)))) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_mean_of_values(causal):
    rng = np.random.default_rng(1)
    n, d = 37, 8
    q = np.zeros((n, d))
    k, v = rnd(rng, n, d), rnd(rng, n, d)
    o, lse = attention_fwd_head(q, k, v, 0.35, causal)
    for i in range(n):
        cnt = i + 1 if causal else n
        np.testing.assert_allclose(o[i], v[:cnt].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[i] - math.log(cnt)) <= 1e-13


def test_single_key():
    rng = np.random.default_rng(2)
    for causal in (False, True):
        q, k, v = rnd(rng, 1, 5), rnd(rng, 1, 5), rnd(rng, 1, 5)
        o, lse = attention_fwd_head(q, k, v, 0.5, causal)
        np.testing.assert_array_equal(o, v)
        assert abs(lse[0] - 0.5 * float(q[0] @ k[0])) <= 1e-15


def test_causal_row_zero_is_first_value_row():
    rng = np.random.default_rng(3)
    q, k, v = rnd(rng, 20, 6, s=3), rnd(rng, 20, 6, s=3), rnd(rng, 20, 6)
    o, lse = attention_fwd_head(q, k, v, 0.4, True)
    np.testing.assert_array_equal(o[0], v[0])
    assert abs(lse[0] - 0.4 * float(q[0] @ k[0])) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_and_rows_sum_to_one(causal):
    rng = np.random.default_rng(4)
    n, d = 50, 16
    q, k = rnd(rng, n, d, s=2), rnd(rng, n, d, s=2)
    c = rnd(rng, d)
    o, _ = attention_fwd_head(q, k, np.tile(c, (n, 1)), 0.25, causal)
    np.testing.assert_allclose(o, np.tile(c, (n, 1)), rtol=0, atol=1e-13)
    o1, _ = attention_fwd_head(q, k, np.ones((n, d)), 0.25, causal)
    np.testing.assert_allclose(o1, 1.0, rtol=0, atol=1e-14)


def test_dominant_key_selects_its_value():
    """A key aligned with the query at a huge scale takes all the weight."""
    rng = np.random.default_rng(5)
    n, d = 16, 4
    q = np.zeros((n, d)); q[:, 0] = 1.0
    k = rnd(rng, n, d) * 0.01
    k[9, 0] = 1.0
    v = rnd(rng, n, d)
    o, lse = attention_fwd_head(q, k, v, 1e4, False)
    np.testing.assert_allclose(o, np.tile(v[9], (n, 1)), atol=1e-12)
    np.testing.assert_allclose(lse, 1e4, rtol=1e-12)


# ---------------------------------------------------------------- invariants

def test_key_shift_invariance():
    rng = np.random.default_rng(6)
    n, d, sc = 40, 8, 0.3
    q, k, v = rnd(rng, n, d), rnd(rng, n, d), rnd(rng, n, d)
    c = rnd(rng, d)
    for causal in (False, True):
        o, l = attention_fwd_head(q, k, v, sc, causal)
        o2, l2 = attention_fwd_head(q, k + c, v, sc, causal)
        np.testing.assert_allclose(o2, o, atol=1e-12)
        np.testing.assert_allclose(l2, l + sc * (q @ c), atol=1e-12)


def test_joint_key_value_permutation_noncausal():
    rng = np.random.default_rng(7)
    n, d = 33, 8
    q, k, v = rnd(rng, n, d), rnd(rng, n, d), rnd(rng, n, d)
    perm = rng.permutation(n)
    o, l = attention_fwd_head(q, k, v, 0.3, False)
    o2, l2 = attention_fwd_head(q, k[perm], v[perm], 0.3, False)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(l2, l, atol=1e-13)


def test_query_permutation_noncausal():
    rng = np.random.default_rng(8)
    n, d = 33, 8
    q, k, v = rnd(rng, n, d), rnd(rng, n, d), rnd(rng, n, d)
    perm = rng.permutation(n)
    o, l = attention_fwd_head(q, k, v, 0.3, False)
    o2, l2 = attention_fwd_head(q[perm], k, v, 0.3, False)
    np.testing.assert_allclose(o2, o[perm], atol=1e-13)
    np.testing.assert_allclose(l2, l[perm], atol=1e-13)


def test_linear_in_values():
    rng = np.random.default_rng(9)
    n, d = 30, 8
    q, k, v1, v2 = (rnd(rng, n, d) for _ in range(4))
    for causal in (False, True):
        a, _ = attention_fwd_head(q, k, v1, 0.3, causal)
        b, _ = attention_fwd_head(q, k, v2, 0.3, causal)
        c, _ = attention_fwd_head(q, k, 2.0 * v1 - 3.0 * v2, 0.3, causal)
        np.testing.assert_allclose(c, 2.0 * a - 3.0 * b, atol=1e-12)


def test_causal_last_row_change_only_affects_last_output():
    rng = np.random.default_rng(10)
    n, d = 25, 8
    q, k, v = rnd(rng, n, d), rnd(rng, n, d), rnd(rng, n, d)
    o, l = attention_fwd_head(q, k, v, 0.3, True)
    k2, v2 = k.copy(), v.copy()
    k2[-1] += 5.0
    v2[-1] -= 3.0
    o2, l2 = attention_fwd_head(q, k2, v2, 0.3, True)
    np.testing.assert_array_equal(o2[:-1], o[:-1])
    np.testing.assert_array_equal(l2[:-1], l[:-1])
    assert np.max(np.abs(o2[-1] - o[-1])) > 1e-3


def test_batched_heads_are_independent_and_match_per_head():
    rng = np.random.default_rng(11)
    q, k, v = (rnd(rng, 2, 3, 19, 4) for _ in range(3))
    o, l = attention_fwd(q, k, v, 0.5, True)
    for b in range(2):
        for h in range(3):
            oh, lh = attention_fwd_head(q[b, h], k[b, h], v[b, h], 0.5, True)
            np.testing.assert_array_equal(o[b, h], oh)
            np.testing.assert_array_equal(l[b, h], lh)


def test_sampled_rows_equal_full_rows_and_chunking(monkeypatch):
    rng = np.random.default_rng(12)
    n, d = 300, 8
    q, k, v = rnd(rng, n, d), rnd(rng, n, d), rnd(rng, n, d)
    for causal in (False, True):
        o, l = attention_fwd_head(q, k, v, 0.3, causal)
        rows = np.array([0, 1, 7, 128, 255, 299])
        os_, ls = attention_fwd_head(q, k, v, 0.3, causal, rows=rows)
        np.testing.assert_allclose(os_, o[rows], atol=1e-14)
        np.testing.assert_allclose(ls, l[rows], atol=1e-14)
        monkeypatch.setattr(oatt, "ROW_CHUNK", 64)
        o3, l3 = attention_fwd_head(q, k, v, 0.3, causal)
        monkeypatch.undo()
        np.testing.assert_allclose(o3, o, atol=1e-14)
        np.testing.assert_allclose(l3, l, atol=1e-14)


def test_large_scores_do_not_overflow():
    rng = np.random.default_rng(13)
    n, d = 64, 16
    q, k, v = rnd(rng, n, d, s=30), rnd(rng, n, d, s=30), rnd(rng, n, d)
    o, l = attention_fwd_head(q, k, v, 1.0, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


# ---------------------------------------------------------------- backward

def _loss(q, k, v, do, scale, causal):
    o, _ = attention_fwd_head(q, k, v, scale, causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sc", [0.7, -0.45])
def test_backward_matches_central_finite_differences(causal, sc):
    rng = np.random.default_rng(20 + causal)
    n, d = 6, 3
    q, k, v, do = (rnd(rng, n, d) for _ in range(4))
    dq, dk, dv = attention_bwd_head(q, k, v, do, sc, causal)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, sc, causal)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], do, sc, causal)) / (2 * h)
        err = np.max(np.abs(num - g)) / max(1.0, np.max(np.abs(g)))
        assert err <= 1e-7, (name, err)


def test_backward_constant_values_gives_zero_dq_dk():
    rng = np.random.default_rng(22)
    n, d = 40, 8
    q, k, do = rnd(rng, n, d), rnd(rng, n, d), rnd(rng, n, d)
    v = np.tile(rnd(rng, d), (n, 1))
    for causal in (False, True):
        dq, dk, dv = attention_bwd_head(q, k, v, do, 0.3, causal)
        assert np.max(np.abs(dq)) <= 1e-12 and np.max(np.abs(dk)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_backward_sum_identities(causal):
    """sum_j dK_j = 0 (key-shift invariance); sum_j dV_j = sum_i dO_i (rows of P sum to 1)."""
    rng = np.random.default_rng(23)
    n, d = 45, 8
    q, k, v, do = (rnd(rng, n, d) for _ in range(4))
    dq, dk, dv = attention_bwd_head(q, k, v, do, 0.3, causal)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)


def test_backward_single_query_row_closed_form():
    """One query, non-causal: dV_j = p_j dO, dQ = scale * sum_j p_j (dO.v_j - dO.o) k_j."""
    rng = np.random.default_rng(24)
    n, d, sc = 9, 5, 0.6
    q, k, v, do = rnd(rng, 1, d), rnd(rng, n, d), rnd(rng, n, d), rnd(rng, 1, d)
    # The oracle takes equal query/key lengths; pad the queries with zero-gradient rows.
    qp = np.vstack([q, np.zeros((n - 1, d))])
    dop = np.vstack([do, np.zeros((n - 1, d))])
    dq, dk, dv = attention_bwd_head(qp, k, v, dop, sc, False)
    s = sc * (k @ q[0])
    p = np.exp(s - s.max()); p /= p.sum()
    o = p @ v
    np.testing.assert_allclose(dv, np.outer(p, do[0]), atol=1e-14)
    g = p * (v @ do[0] - do[0] @ o)
    np.testing.assert_allclose(dq[0], sc * (g @ k), atol=1e-14)
    np.testing.assert_allclose(dk, sc * np.outer(g, q[0]), atol=1e-14)


def test_cross_check_with_torch_float64_autograd():
    """Independent implementation (torch CPU float64 ops + autograd) on a
    moderate shape: a cross-check only, never used as the oracle."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(25)
    n, d, sc = 70, 16, 0.25
    q, k, v, do = (rnd(rng, n, d) for _ in range(4))
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        s = sc * tq @ tk.T
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv
        lse = torch.logsumexp(s, dim=-1)
        o.backward(torch.tensor(do))
        oo, ol = attention_fwd_head(q, k, v, sc, causal)
        np.testing.assert_allclose(oo, o.detach().numpy(), atol=1e-13)
        np.testing.assert_allclose(ol, lse.detach().numpy(), atol=1e-13)
        dq, dk, dv = attention_bwd_head(q, k, v, do, sc, causal)
        np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


# ---------------------------------------------------------------- mutation check

def _pins_pass(mod) -> bool:
    """Run a compact battery of the pins above against module ``mod``.

    Comparisons are written as ``not err <= tol`` so that a NaN counts as a failure."""
    rng = np.random.default_rng(31)
    try:
        for causal in (False, True):
            n, d = 5, 3
            q, k, v = rnd(rng, n, d, s=1.5), rnd(rng, n, d, s=1.5), rnd(rng, n, d)
            sc = 0.6
            o, lse = mod.attention_fwd_head(q, k, v, sc, causal)
            ob, lb = brute_fwd_decimal(q, k, v, sc, causal)
            if not np.max(np.abs(o - np.array([[float(x) for x in r] for r in ob]))) <= 1e-12:
                return False
            if not np.max(np.abs(lse - np.array([float(x) for x in lb]))) <= 1e-12:
                return False
            do = rnd(rng, n, d)
            dq, dk, dv = mod.attention_bwd_head(q, k, v, do, sc, causal)
            h = 1e-6
            for which, g in ((0, dq), (1, dk), (2, dv)):
                args = [q, k, v]
                for idx in np.ndindex(n, d):
                    ap = [a.copy() for a in args]
                    am = [a.copy() for a in args]
                    ap[which][idx] += h
                    am[which][idx] -= h
                    lp = float(np.sum(mod.attention_fwd_head(*ap, sc, causal)[0] * do))
                    lm = float(np.sum(mod.attention_fwd_head(*am, sc, causal)[0] * do))
                    if not abs((lp - lm) / (2 * h) - g[idx]) <= 1e-6:
                        return False
        return True
    except Exception:
        return False


MUTATIONS = [
    ("drop scale in scores", "s = scale * (q_rows @ k[:nk].T)", "s = (q_rows @ k[:nk].T)"),
    ("keys in reversed order", "s = scale * (q_rows @ k[:nk].T)", "s = scale * (q_rows @ k[:nk][::-1].T)"),
    ("causal off by one", "np.arange(nk)[None, :] <= rows[:, None]", "np.arange(nk)[None, :] < rows[:, None]"),
    ("causal mask reversed", "np.arange(nk)[None, :] <= rows[:, None]", "np.arange(nk)[None, :] >= rows[:, None]"),
    ("lse drops the max", "lse = (m + np.log(z))[:, 0]", "lse = (np.log(z))[:, 0]"),
    ("softmax not normalised", "p = e / z", "p = e"),
    ("output uses transposed P", "o[c0:c0 + r.shape[0]] = p @ v[:nk]", "o[c0:c0 + r.shape[0]] = p.T @ v[:nk]"),
    ("dV uses transposed P", "dv[:nk] += p.T @ g", "dv[:nk] += p @ g"),
    ("dP transposed", "dp = g @ v[:nk].T", "dp = v[:nk] @ g.T"),
    ("Jacobian sign", "ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * (dp + (p * dp).sum(axis=1, keepdims=True))"),
    ("Jacobian drops row term", "ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    ("Jacobian sums the wrong axis", "ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * (dp - (p * dp).sum(axis=0, keepdims=True))"),
    ("dQ missing scale", "dq[r] = scale * (ds @ k[:nk])", "dq[r] = (ds @ k[:nk])"),
    ("dK uses keys", "dk[:nk] += scale * (ds.T @ q[r])", "dk[:nk] += scale * (ds.T @ k[r])"),
]


def test_unmutated_oracle_passes_battery():
    assert _pins_pass(oatt)


@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutations_are_caught(label, old, new):
    src = open(oatt.__file__).read()
    assert old in src, f"mutation anchor not found: {label}"
    mutated = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(mutated, "<mutant>", "exec"), mod.__dict__)
    assert not _pins_pass(mod), f"pins did not catch mutation: {label}"
