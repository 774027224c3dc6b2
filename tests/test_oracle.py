"""CPU pins of the float64 oracle against what the pages and mathematics fix.

None of these tests re-types the oracle's own formula: each compares it with
a different route to the same answer (hand-derived closed forms, brute-force
support enumeration, an independent bisection, the variational objective,
a numerical optimiser, finite differences, direct definitions of the masks).
"""

import itertools
import math
import os
import re

import numpy as np
import pytest

from oracle import (
    allowed_mask,
    attention_backward,
    entmax15_backward,
    attention_forward,
    entmax15_bisect,
    entmax15_exact,
    tsallis15_objective,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "entmax15_closed_forms.txt")
_EXPR_OK = re.compile(r"^[0-9+\-*/(). sqrt]+$")


def _eval(expr):
    assert _EXPR_OK.match(expr), expr
    return float(eval(expr, {"__builtins__": {}}, {"sqrt": math.sqrt}))


def _golden_cases():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fields = dict(part.strip().split("=", 1) for part in line.split(";"))
            fields = {k.strip(): v.strip() for k, v in fields.items()}
            s = np.array([float(x) for x in fields["s"].split()])
            tau = _eval(fields["tau"])
            p = np.array([_eval(x) for x in fields["p"].split()])
            cases.append((s, tau, p))
    return cases


# ---------------------------------------------------------------------------
# Closed forms (Theorem 1, hand-derived)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: str(c[0].tolist()))
def test_golden_closed_forms(case):
    s, tau, p = case
    p_o, tau_o = entmax15_exact(s)
    assert tau_o == pytest.approx(tau, abs=1e-13)
    np.testing.assert_allclose(p_o, p, atol=1e-13)


def test_single_entry():
    for s0 in (-3.0, 0.0, 7.25):
        p, tau = entmax15_exact(np.array([s0]))
        assert p[0] == 1.0 and tau == pytest.approx(s0 - 2.0, abs=1e-14)


def test_two_entries_closed_form():
    # t = s1 - s2 in [0, 2): p1 = ((t + sqrt(8 - t^2))/4)^2; t >= 2: one-hot
    rng = np.random.default_rng(1)
    for _ in range(200):
        s2 = rng.normal()
        t = rng.uniform(0, 3)
        s = np.array([s2 + t, s2])
        p, tau = entmax15_exact(s)
        if t < 2:
            p1 = ((t + math.sqrt(8 - t * t)) / 4) ** 2
            tau_ref = (s[0] + s[1]) / 2 - math.sqrt(2 - t * t / 4)
        else:
            p1, tau_ref = 1.0, s[0] - 2.0
        assert p[0] == pytest.approx(p1, abs=1e-12)
        assert p[1] == pytest.approx(1 - p1, abs=1e-12)
        assert tau == pytest.approx(tau_ref, abs=1e-12)


def test_uniform_row_hits_upper_bracket():
    # equal scores: p = 1/n and tau = s - 2/sqrt(n), the top of the bracket
    # [max - 2, max - 2/sqrt(n)] ("DistilBERT SST-2 with AdaSplash
    # Attention", Mathematical Formulation 2)
    for n in (1, 2, 3, 7, 64, 1000):
        s = np.full(n, 0.3)
        p, tau = entmax15_exact(s)
        np.testing.assert_allclose(p, 1.0 / n, atol=1e-14)
        assert tau == pytest.approx(0.3 - 2 / math.sqrt(n), abs=1e-13)


def test_gap_of_two_is_one_hot():
    rng = np.random.default_rng(2)
    for _ in range(100):
        n = rng.integers(2, 20)
        s = rng.normal(size=n)
        i = rng.integers(n)
        s[i] = np.max(np.delete(s, i)) + 2.0 + rng.uniform(0, 3)
        p, tau = entmax15_exact(s)
        assert p[i] == 1.0 and np.count_nonzero(p) == 1


# ---------------------------------------------------------------------------
# Invariants (Theorem 1, KKT; bracket of the DistilBERT card)
# ---------------------------------------------------------------------------

def _rows(rng, n_rows=60):
    rows = []
    for _ in range(n_rows):
        n = int(rng.integers(1, 300))
        scale = float(rng.choice([0.05, 0.3, 1.0, 3.0, 20.0]))
        rows.append(rng.normal(size=n) * scale + rng.normal() * 5)
    return rows


def test_simplex_kkt_and_bracket():
    rng = np.random.default_rng(3)
    for s in _rows(rng):
        p, tau = entmax15_exact(s)
        assert np.all(p >= 0)
        assert p.sum() == pytest.approx(1.0, abs=1e-12)
        supp = p > 0
        # on the support 2 sqrt(p) = s - tau, off it s <= tau
        np.testing.assert_allclose(2 * np.sqrt(p[supp]), s[supp] - tau, atol=1e-11)
        assert np.all(s[~supp] <= tau + 1e-12)
        m, n = s.max(), s.size
        assert m - 2 - 1e-12 <= tau <= m - 2 / math.sqrt(n) + 1e-12


def test_shift_and_permutation():
    rng = np.random.default_rng(4)
    for s in _rows(rng, 30):
        p, tau = entmax15_exact(s)
        c = rng.normal() * 10
        p2, tau2 = entmax15_exact(s + c)
        np.testing.assert_allclose(p2, p, atol=1e-12)
        assert tau2 == pytest.approx(tau + c, abs=1e-10)
        perm = rng.permutation(s.size)
        p3, tau3 = entmax15_exact(s[perm])
        np.testing.assert_allclose(p3, p[perm], atol=1e-13)
        assert tau3 == pytest.approx(tau, abs=1e-12)


def test_masked_entries_are_excluded():
    # entmax over an allowed subset equals entmax of the sub-vector, with
    # exact zeros on the disallowed entries
    rng = np.random.default_rng(5)
    for _ in range(50):
        n = int(rng.integers(2, 100))
        s = rng.normal(size=n)
        ok = rng.random(n) < 0.6
        ok[rng.integers(n)] = True
        p, tau = entmax15_exact(s, ok)
        p_sub, tau_sub = entmax15_exact(s[ok])
        np.testing.assert_allclose(p[ok], p_sub, atol=1e-14)
        assert np.all(p[~ok] == 0) and tau == tau_sub


def test_empty_row():
    p, tau = entmax15_exact(np.array([[1.0, 2.0]]), np.array([[False, False]]))
    assert np.all(p == 0) and np.isinf(tau[0])


# ---------------------------------------------------------------------------
# Brute force over all supports (tiny rows)
# ---------------------------------------------------------------------------

def _brute_force(s):
    """Enumerate every non-empty support; keep the one meeting the KKT
    conditions of Theorem 1.  Written without sorting or prefix sums."""
    n = s.size
    found = []
    for r in range(1, n + 1):
        for sub in itertools.combinations(range(n), r):
            idx = list(sub)
            vals = s[idx]
            # solve sum (v - tau)^2 = 4: r tau^2 - 2 tau sum v + (sum v^2 - 4) = 0
            a, b, c = r, -2 * vals.sum(), (vals ** 2).sum() - 4
            disc = b * b - 4 * a * c
            if disc < 0:
                continue
            tau = (-b - math.sqrt(disc)) / (2 * a)
            others = np.delete(s, idx)
            if np.all(vals > tau) and np.all(others <= tau):
                found.append((tau, idx))
    return found


def test_brute_force_supports():
    rng = np.random.default_rng(6)
    for _ in range(300):
        n = int(rng.integers(1, 9))
        s = rng.normal(size=n) * rng.choice([0.2, 1.0, 2.5])
        found = _brute_force(s)
        assert len(found) == 1, found          # the KKT point is unique
        tau_bf, idx = found[0]
        p, tau = entmax15_exact(s)
        assert tau == pytest.approx(tau_bf, abs=1e-12)
        assert sorted(np.flatnonzero(p > 0).tolist()) == sorted(idx)


# ---------------------------------------------------------------------------
# Independent bisection (Theorem 2; bracket of the DistilBERT card)
# ---------------------------------------------------------------------------

def test_bisection_agrees_within_its_bound():
    rng = np.random.default_rng(7)
    for s in _rows(rng, 80):
        p, tau = entmax15_exact(s)
        pb, taub = entmax15_bisect(s, n_iter=25)
        width = 2 - 2 / math.sqrt(s.size)
        # 25 halvings of a bracket narrower than 2: error below 2^-25 ~ 3e-8
        assert abs(taub - tau) <= width * 2.0 ** -25 + 1e-12
        assert abs(taub - tau) < 3e-8
        p60, tau60 = entmax15_bisect(s, n_iter=60)
        assert tau60 == pytest.approx(tau, abs=1e-12)
        np.testing.assert_allclose(p60, p, atol=1e-11)


# ---------------------------------------------------------------------------
# Variational definition (section 2.1): p maximises p.s + H_1.5(p)
# ---------------------------------------------------------------------------

def test_variational_optimality_pairwise_moves():
    rng = np.random.default_rng(8)
    for _ in range(40):
        n = int(rng.integers(2, 12))
        s = rng.normal(size=n)
        p, _ = entmax15_exact(s)
        f0 = tsallis15_objective(p, s)
        for a in range(n):
            for b in range(n):
                if a == b or p[b] == 0:
                    continue
                eps = min(1e-3, p[b])
                q = p.copy()
                q[a] += eps
                q[b] -= eps
                assert tsallis15_objective(q, s) <= f0 + 1e-14
        for _ in range(50):
            q = rng.dirichlet(np.ones(n) * rng.choice([0.1, 1.0, 10.0]))
            assert tsallis15_objective(q, s) <= f0 + 1e-12


def test_matches_numerical_optimiser():
    scipy_opt = pytest.importorskip("scipy.optimize")
    rng = np.random.default_rng(9)
    for _ in range(10):
        n = int(rng.integers(2, 8))
        s = rng.normal(size=n)
        res = scipy_opt.minimize(
            lambda x: -tsallis15_objective(np.clip(x, 0, None), s),
            np.full(n, 1.0 / n), method="SLSQP", bounds=[(0, 1)] * n,
            constraints=[{"type": "eq", "fun": lambda x: x.sum() - 1}],
            options={"ftol": 1e-14, "maxiter": 500})
        p, _ = entmax15_exact(s)
        np.testing.assert_allclose(res.x, p, atol=2e-5)


# ---------------------------------------------------------------------------
# Masks (section 3 of the AdaSplash page; window as i - W < j <= i)
# ---------------------------------------------------------------------------

def test_allowed_mask_definitions():
    L, W = 70, 32
    a = allowed_mask(L, causal=True, window=W)
    for i in range(L):
        for j in range(L):
            assert a[i, j] == (i - W < j <= i)
    assert list(a.sum(1)) == [min(i + 1, W) for i in range(L)]
    c = allowed_mask(L, causal=True)
    assert np.array_equal(c, np.tril(np.ones((L, L), bool)))
    km = (np.arange(L) < 17).astype(np.uint8)
    m = allowed_mask(L, km)
    assert np.all(m[:, :17]) and not np.any(m[:, 17:])
    with pytest.raises(ValueError):
        allowed_mask(L, window=4)


def test_large_negative_fill_matches_exclusion():
    # The page code fills masked logits with -10000 before entmax; while an
    # allowed score exceeds -9998 that fill gives exactly zero weight, so it
    # agrees with excluding the key from the simplex.
    rng = np.random.default_rng(10)
    s = rng.normal(size=(40, 40)) * 3
    ok = allowed_mask(40, (rng.random(40) < 0.7).astype(np.uint8), causal=True)
    ok[:, 0] = True
    p_ex, tau_ex = entmax15_exact(s, ok)
    p_fill, _ = entmax15_exact(np.where(ok, s, -10000.0))
    np.testing.assert_allclose(p_fill, p_ex, atol=1e-13)


# ---------------------------------------------------------------------------
# Attention forward: scores, scale, aggregation
# ---------------------------------------------------------------------------

def test_attention_forward_small_loops():
    rng = np.random.default_rng(11)
    B, H, L, d = 1, 2, 9, 4
    q, k, v = (rng.normal(size=(B, H, L, d)) for _ in range(3))
    km = np.array([[1, 1, 1, 0, 1, 1, 1, 1, 0]], dtype=np.uint8)
    res = attention_forward(q, k, v, km, causal=True, return_probs=True)
    for hh in range(H):
        for i in range(L):
            js = [j for j in range(L) if km[0, j] and j <= i]
            if not js:
                assert np.all(res["out"][hh, i] == 0) and np.isinf(res["tau"][hh, i])
                continue
            s = np.array([sum(q[0, hh, i, t] * k[0, hh, j, t] for t in range(d)) / math.sqrt(d) for j in js])
            found = _brute_force(s)
            tau = found[0][0]
            p = np.maximum((s - tau) / 2, 0) ** 2
            o = sum(p[a] * v[0, hh, j] for a, j in enumerate(js))
            np.testing.assert_allclose(res["out"][hh, i], o, atol=1e-12)
            assert res["tau"][hh, i] == pytest.approx(tau, abs=1e-12)
            assert res["probs"][hh, i].sum() == pytest.approx(1.0, abs=1e-12)


def test_attention_rows_subset_matches_full():
    rng = np.random.default_rng(12)
    q, k, v = (rng.normal(size=(2, 2, 33, 8)) for _ in range(3))
    full = attention_forward(q, k, v)
    rows = np.array([0, 5, 32])
    part = attention_forward(q, k, v, rows=rows, heads=[(1, 0), (0, 1)])
    np.testing.assert_allclose(part["out"][0], full["out"][2][rows])
    np.testing.assert_allclose(part["tau"][1], full["tau"][1][rows])


# ---------------------------------------------------------------------------
# Backward: finite differences (section 2.4 Jacobian)
# ---------------------------------------------------------------------------

def _loss(q, k, v, dout, **kw):
    return float((attention_forward(q, k, v, **kw)["out"] * dout).sum())


@pytest.mark.parametrize("kw", [{}, {"causal": True}, {"causal": True, "window": 3},
                                {"key_mask": np.array([[1, 1, 0, 1, 1, 0, 1]], np.uint8)}])
def test_backward_finite_differences(kw):
    rng = np.random.default_rng(13)
    B, H, L, d = 1, 1, 7, 3
    q, k, v, do = (rng.normal(size=(B, H, L, d)) for _ in range(4))
    q *= 1.5
    g = attention_backward(q, k, v, do, **kw)
    h = 1e-6
    for name, x, ref in (("q", q, g["dq"]), ("k", k, g["dk"]), ("v", v, g["dv"])):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, **kw)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, **kw)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(ref[0], num[0, 0], atol=2e-7, err_msg=name)


def test_jacobian_identities():
    # J_ij = sqrt(p_i)(delta_ij - sqrt(p_j)/sum sqrt(p)) on the support:
    # symmetric, annihilates constants, zero off the support.  Built from
    # finite differences of the exact map (not from the closed form).
    rng = np.random.default_rng(14)
    for _ in range(10):
        n = int(rng.integers(2, 10))
        s = rng.normal(size=n)
        h = 1e-7
        J = np.zeros((n, n))
        for j in range(n):
            e = np.zeros(n); e[j] = h
            J[:, j] = (entmax15_exact(s + e)[0] - entmax15_exact(s - e)[0]) / (2 * h)
        p, _ = entmax15_exact(s)
        np.testing.assert_allclose(J, J.T, atol=1e-6)
        np.testing.assert_allclose(J @ np.ones(n), 0, atol=1e-6)
        off = p == 0
        assert np.all(np.abs(J[off]) < 1e-6) and np.all(np.abs(J[:, off]) < 1e-6)
        w = np.sqrt(p)
        J_closed = np.diag(w) - np.outer(w, w) / w.sum()
        np.testing.assert_allclose(J, J_closed, atol=1e-6)


def test_grouped_query_forward_equals_repeated_heads():
    # "ADASPLASH -- ROBERTA Benchmark Result", section 3: with H_kv < H the
    # key/value heads are repeated (each for H / H_kv consecutive query
    # heads) before the scores; the oracle takes k, v with H_kv heads.
    rng = np.random.default_rng(21)
    B, H, Hkv, L, d = 2, 6, 2, 9, 4
    q = rng.normal(size=(B, H, L, d)) * 1.3
    k, v = rng.normal(size=(B, Hkv, L, d)), rng.normal(size=(B, Hkv, L, d))
    km = (rng.random((B, L)) > 0.2).astype(np.uint8)
    for kw in ({}, {"key_mask": km}, {"causal": True, "window": 4}):
        g = attention_forward(q, k, v, **kw)
        r = attention_forward(q, np.repeat(k, H // Hkv, axis=1), np.repeat(v, H // Hkv, axis=1), **kw)
        np.testing.assert_allclose(g["out"], r["out"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(g["tau"], r["tau"], rtol=0, atol=1e-13)
    # distinct heads of a group see the same keys but give different rows
    assert not np.allclose(g["out"][0], g["out"][1])


def test_grouped_query_backward_finite_differences():
    # the gradient of a shared key/value head sums the query heads of its
    # group: checked against central differences of the forward
    rng = np.random.default_rng(22)
    B, H, Hkv, L, d = 1, 4, 2, 6, 3
    q = rng.normal(size=(B, H, L, d)) * 1.4
    k, v = rng.normal(size=(B, Hkv, L, d)), rng.normal(size=(B, Hkv, L, d))
    do = rng.normal(size=(B, H, L, d))
    g = attention_backward(q, k, v, do, causal=True)
    h = 1e-6
    for name, x, ref in (("k", k, g["dk_kv"]), ("v", v, g["dv_kv"])):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"k": k, "v": v}
            args[name] = xp
            fp = _loss(q, args["k"], args["v"], do, causal=True)
            args[name] = xm
            fm = _loss(q, args["k"], args["v"], do, causal=True)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(ref, num, atol=3e-7, err_msg=name)
    dqn = np.zeros_like(q)
    for idx in np.ndindex(*q.shape):
        xp = q.copy(); xp[idx] += h
        xm = q.copy(); xm[idx] -= h
        dqn[idx] = (_loss(xp, k, v, do, causal=True) - _loss(xm, k, v, do, causal=True)) / (2 * h)
    np.testing.assert_allclose(g["dq"], dqn[0], atol=3e-7)


def test_row_backward_matches_finite_differences():
    # ds = J^T dp with J the Jacobian of the exact map, built here by central
    # differences of entmax15_exact (not from the closed form)
    rng = np.random.default_rng(23)
    for _ in range(8):
        n = int(rng.integers(2, 12))
        s = rng.normal(size=n) * 1.5
        allowed = rng.random(n) > 0.25
        allowed[0] = True
        dp = rng.normal(size=n)
        h = 1e-7
        J = np.zeros((n, n))
        for j in range(n):
            e = np.zeros(n); e[j] = h
            J[:, j] = (entmax15_exact(s + e, allowed)[0] - entmax15_exact(s - e, allowed)[0]) / (2 * h)
        np.testing.assert_allclose(entmax15_backward(s, dp, allowed), J.T @ dp, atol=2e-6)
    # an empty row has no gradient
    assert np.all(entmax15_backward(np.zeros((1, 4)), np.ones((1, 4)), np.zeros((1, 4), bool)) == 0)



def test_exact_handles_tied_scores():
    # low-precision score rows repeat values, so whole tie groups can sit at
    # the support boundary; the result must still agree with an independent
    # bisection and sum to one
    rng = np.random.default_rng(24)
    s = rng.normal(size=(200, 512))
    s = np.round(s * 16) / 16           # heavy ties (4 fractional bits)
    p, tau = entmax15_exact(s)
    _, tb = entmax15_bisect(s, n_iter=60)
    np.testing.assert_allclose(tau, tb, atol=1e-10)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)


@pytest.mark.parametrize("window,hkv", [(0, 4), (32, 4), (5, 2), (0, 1)])
def test_decode_is_last_row_of_causal_forward(window, hkv):
    # one new query against a cache = the last row of causal (windowed)
    # attention over the cached prefix, computed through allowed_mask
    from oracle import attention_decode, attention_forward
    rng = np.random.default_rng(window + 10 * hkv)
    B, H, S, d = 4, 4, 70, 16
    q = rng.normal(size=(B, H, d))
    kc = rng.normal(size=(B, hkv, S, d))
    vc = rng.normal(size=(B, hkv, S, d))
    seqlens = np.array([S, 1, 37, 0])
    out, tau = attention_decode(q, kc, vc, seqlens, window)
    assert np.all(out[3] == 0) and np.all(np.isinf(tau[3]))
    for b in range(3):
        n = seqlens[b]
        qf = rng.normal(size=(1, H, n, d))
        qf[0, :, n - 1] = q[b]
        ref = attention_forward(qf, kc[b:b + 1, :, :n], vc[b:b + 1, :, :n], causal=True, window=window,
                                rows=[n - 1])
        np.testing.assert_allclose(out[b], ref["out"][:, 0], atol=1e-12)
        np.testing.assert_allclose(tau[b], ref["tau"][:, 0], atol=1e-12)


def test_decode_window_one_is_own_value():
    # W = 1: only the query's own key; p = 1 there, so O = v_own and
    # ((s - tau)/2)^2 = 1 gives tau = s - 2
    from oracle import attention_decode
    rng = np.random.default_rng(2)
    q = rng.normal(size=(2, 3, 8))
    kc = rng.normal(size=(2, 3, 10, 8))
    vc = rng.normal(size=(2, 3, 10, 8))
    out, tau = attention_decode(q, kc, vc, [10, 4], window=1)
    for b, n in ((0, 10), (1, 4)):
        for h in range(3):
            np.testing.assert_allclose(out[b, h], vc[b, h, n - 1], atol=1e-14)
            s = q[b, h] @ kc[b, h, n - 1] / np.sqrt(8)
            assert abs(tau[b, h] - (s - 2.0)) < 1e-12


@pytest.mark.parametrize("window,hkv", [(0, 2), (6, 4)])
def test_decode_several_queries_are_the_last_rows_of_causal_forward(window, hkv):
    # Lq new queries at the end of each cached sequence = the last Lq rows
    # of causal (windowed) attention over the prefix; a sequence shorter than
    # Lq leaves its first queries without keys
    from oracle import attention_decode, attention_forward
    rng = np.random.default_rng(40 + window)
    B, H, S, d, Lq = 3, 4, 50, 16, 5
    q = rng.normal(size=(B, H, Lq, d))
    kc = rng.normal(size=(B, hkv, S, d))
    vc = rng.normal(size=(B, hkv, S, d))
    seqlens = np.array([S, 23, 3])
    out, tau = attention_decode(q, kc, vc, seqlens, window)
    for b in range(B):
        n = seqlens[b]
        qf = rng.normal(size=(1, H, n, d))
        m = min(n, Lq)
        qf[0, :, n - m:] = q[b, :, Lq - m:]
        ref = attention_forward(qf, kc[b:b + 1, :, :n], vc[b:b + 1, :, :n], causal=True, window=window,
                                rows=np.arange(n - m, n))
        np.testing.assert_allclose(out[b, :, Lq - m:], ref["out"], atol=1e-12)
        np.testing.assert_allclose(tau[b, :, Lq - m:], ref["tau"], atol=1e-12)
        assert np.all(out[b, :, :Lq - m] == 0) and np.all(np.isinf(tau[b, :, :Lq - m]))


def test_decode_without_causal_mask_is_full_attention_over_the_cache():
    # causal=False: every cached key for every query, i.e. the bidirectional
    # forward of the queries against the n cached keys (rows of a longer
    # sequence whose keys past n are padding)
    from oracle import attention_decode, attention_forward
    rng = np.random.default_rng(9)
    B, H, S, d, Lq = 2, 2, 30, 8, 4
    q = rng.normal(size=(B, H, Lq, d))
    kc = rng.normal(size=(B, H, S, d))
    vc = rng.normal(size=(B, H, S, d))
    seqlens = np.array([S, 11])
    out, tau = attention_decode(q, kc, vc, seqlens, 0, causal=False)
    for b in range(B):
        n = seqlens[b]
        qf = np.zeros((1, H, S, d))
        qf[0, :, :Lq] = q[b]
        km = (np.arange(S) < n).astype(np.uint8)[None, :]
        ref = attention_forward(qf, kc[b:b + 1], vc[b:b + 1], key_mask=km, rows=np.arange(Lq))
        np.testing.assert_allclose(out[b], ref["out"], atol=1e-12)
        np.testing.assert_allclose(tau[b], ref["tau"], atol=1e-12)
    with pytest.raises(ValueError):
        attention_decode(q, kc, vc, seqlens, 4, causal=False)


# ---------------------------------------------------------------------------
# Backward at query length below key length (decode form)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal,window", [(True, 0), (True, 3), (False, 0)])
def test_decode_backward_finite_differences(causal, window):
    # central differences of attention_decode itself: grouped heads, two
    # sequences of different valid lengths, two queries each
    from oracle import attention_decode, attention_decode_backward
    rng = np.random.default_rng(31 + window + 7 * causal)
    B, H, Hkv, Lq, S, d = 2, 4, 2, 2, 6, 3
    q = rng.normal(size=(B, H, Lq, d)) * 1.4
    kc, vc = rng.normal(size=(B, Hkv, S, d)), rng.normal(size=(B, Hkv, S, d))
    do = rng.normal(size=(B, H, Lq, d))
    seqlens = np.array([S, 4])

    def loss(q_, k_, v_):
        return float((attention_decode(q_, k_, v_, seqlens, window, causal=causal)[0] * do).sum())

    dq, dk, dv = attention_decode_backward(q, kc, vc, do, seqlens, window, causal=causal)
    h = 1e-6
    for x, ref, pos in ((q, dq, 0), (kc, dk, 1), (vc, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            args = [q, kc, vc]
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args[pos] = xp
            fp = loss(*args)
            args[pos] = xm
            fm = loss(*args)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(ref, num, atol=3e-7)
    # keys past the valid length of sequence 1 get no gradient
    assert np.all(dk[1, :, 4:] == 0) and np.all(dv[1, :, 4:] == 0)


def test_decode_backward_is_the_square_backward_when_the_queries_fill_the_cache():
    # Lq = n = S with the causal mask: the decode rows are the causal rows of
    # a square sequence, so the gradients are attention_backward's
    from oracle import attention_backward, attention_decode_backward
    rng = np.random.default_rng(41)
    B, H, L, d = 1, 2, 9, 4
    q, k, v, do = (rng.normal(size=(B, H, L, d)) for _ in range(4))
    for window in (0, 4):
        dq, dk, dv = attention_decode_backward(q, k, v, do, np.array([L]), window, causal=True)
        g = attention_backward(q, k, v, do, causal=True, window=window)
        np.testing.assert_allclose(dq, g["dq"][None], atol=1e-12)
        np.testing.assert_allclose(dk, g["dk"][None], atol=1e-12)
        np.testing.assert_allclose(dv, g["dv"][None], atol=1e-12)
