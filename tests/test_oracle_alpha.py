"""CPU pins of the general-alpha oracle (``oracle/entmax_alpha.py``) against
facts fixed outside it: sparsemax's sort-based closed form at alpha = 2
(Martins and Astudillo 2016, the alpha = 2 case of "ADASPLASH -- ROBERTA
Benchmark Result", section 2.1), the 1.5 closed form of section 2.2 Theorem 1
(itself pinned in test_oracle.py), softmax as alpha goes to 1 (section 2.1),
the variational definition (section 2.1), uniform rows, the bisection error
bound (section 2.3) and finite differences for the backward."""

import numpy as np
import pytest

from oracle import (
    entmax15_backward,
    entmax15_exact,
    entmax_alpha_backward,
    entmax_alpha_vjp,
    entmax_alpha_bisect,
    entmax_alpha_exact,
    tsallis_objective,
)


def _sparsemax(z):
    """Euclidean projection onto the simplex by sorting: k is the largest
    index with 1 + k z_(k) > z_(1) + ... + z_(k), tau = (that sum - 1)/k."""
    zs = np.sort(z)[::-1]
    cs = np.cumsum(zs)
    k = np.arange(1, z.size + 1)
    kk = k[1 + k * zs > cs].max()
    tau = (cs[kk - 1] - 1.0) / kk
    return np.maximum(z - tau, 0.0), tau


def test_sparsemax_worked_example():
    # s = (1, 0.5, -1): support {1, 2}, tau = (1.5 - 1)/2 = 0.25
    p, tau = entmax_alpha_exact(np.array([1.0, 0.5, -1.0]), 2.0)
    np.testing.assert_allclose(p, [0.75, 0.25, 0.0], atol=1e-14)
    assert abs(tau - 0.25) < 1e-14


@pytest.mark.parametrize("seed", range(6))
def test_alpha2_is_sparsemax(seed):
    rng = np.random.default_rng(seed)
    s = rng.normal(size=(5, 40)) * (0.3 + seed)
    p, tau = entmax_alpha_exact(s, 2.0)
    for r in range(s.shape[0]):
        q, t = _sparsemax(s[r])
        np.testing.assert_allclose(p[r], q, atol=1e-12)
        assert abs(tau[r] - t) < 1e-12 * max(1.0, abs(t))


@pytest.mark.parametrize("seed", range(4))
def test_alpha15_matches_closed_form(seed):
    rng = np.random.default_rng(100 + seed)
    s = rng.normal(size=(6, 50)) * (0.5 + 2 * seed)
    allowed = rng.random(s.shape) > 0.3
    p, tau = entmax_alpha_exact(s, 1.5, allowed)
    q, t = entmax15_exact(s, allowed)
    np.testing.assert_allclose(p, q, atol=1e-12)
    np.testing.assert_allclose(tau, t, rtol=1e-12, atol=1e-12)


def test_softmax_limit():
    # alpha -> 1 gives softmax; the gap shrinks in proportion to alpha - 1
    rng = np.random.default_rng(7)
    s = rng.normal(size=30)
    sm = np.exp(s - s.max())
    sm /= sm.sum()
    gaps = []
    for eps in (1e-2, 1e-3):
        p, _ = entmax_alpha_exact(s, 1.0 + eps)
        gaps.append(np.abs(p - sm).max())
    assert gaps[1] < 2e-3
    assert gaps[1] < gaps[0] / 5


@pytest.mark.parametrize("alpha", [1.1, 1.3, 1.5, 1.8, 2.0])
def test_variational_optimality(alpha):
    rng = np.random.default_rng(int(alpha * 100))
    s = rng.normal(size=25) * 2.0
    p, _ = entmax_alpha_exact(s, alpha)
    best = tsallis_objective(p, s, alpha)
    # random points of the simplex, and small feasible moves around p
    for q in rng.dirichlet(np.ones(s.size), size=300):
        assert tsallis_objective(q, s, alpha) <= best + 1e-12
    for _ in range(300):
        d = rng.normal(size=s.size)
        d -= d.mean()
        q = p + 1e-3 * d
        if np.all(q >= 0):
            assert tsallis_objective(q, s, alpha) <= best + 1e-12
    # the other alphas' answers are feasible points too
    for other in (1.2, 1.6, 2.0):
        if other != alpha:
            q, _ = entmax_alpha_exact(s, other)
            assert tsallis_objective(q, s, alpha) <= best + 1e-12


@pytest.mark.parametrize("alpha", [1.05, 1.5, 2.0])
def test_simplex_and_support(alpha):
    rng = np.random.default_rng(3)
    s = rng.normal(size=(8, 64)) * 3.0
    allowed = rng.random(s.shape) > 0.25
    allowed[0] = False
    p, tau = entmax_alpha_exact(s, alpha, allowed)
    assert np.isinf(tau[0]) and np.all(p[0] == 0)
    np.testing.assert_allclose(p[1:].sum(axis=1), 1.0, atol=1e-12)
    assert np.all(p[~allowed] == 0)
    on = allowed[1:] & (s[1:] > tau[1:, None])
    assert np.array_equal(p[1:] > 0, on)


@pytest.mark.parametrize("alpha", [1.2, 1.5, 2.0])
def test_uniform_and_single(alpha):
    p, _ = entmax_alpha_exact(np.full(17, 0.3), alpha)
    np.testing.assert_allclose(p, 1.0 / 17, atol=1e-14)
    allowed = np.zeros(9, dtype=bool)
    allowed[4] = True
    p, _ = entmax_alpha_exact(np.linspace(-1, 1, 9), alpha, allowed)
    np.testing.assert_allclose(p, np.eye(9)[4], atol=1e-14)


@pytest.mark.parametrize("alpha", [1.1, 1.25, 1.5, 1.75, 2.0])
def test_bisection_within_bound(alpha):
    # 25 halvings of [-1, -n^(1-alpha)] in t = (alpha - 1)(tau - max)
    rng = np.random.default_rng(11)
    s = rng.normal(size=(10, 300)) * 2.0
    allowed = rng.random(s.shape) > 0.1
    p, tau = entmax_alpha_bisect(s, alpha, allowed)
    q, t = entmax_alpha_exact(s, alpha, allowed)
    n = allowed.sum(axis=1)
    width = (1.0 - n ** (1.0 - alpha)) / (alpha - 1.0)
    assert np.all(np.abs(tau - t) <= width * 2.0 ** -25 + 1e-12)
    np.testing.assert_allclose(p, q, atol=1e-6)


def _fd_jacobian(s, alpha, h=1e-6):
    J = np.zeros((s.size, s.size))
    for j in range(s.size):
        e = np.zeros(s.size)
        e[j] = h
        J[:, j] = (entmax_alpha_exact(s + e, alpha)[0] - entmax_alpha_exact(s - e, alpha)[0]) / (2 * h)
    return J


@pytest.mark.parametrize("alpha", [1.3, 1.5, 1.9, 2.0])
def test_backward_finite_differences(alpha):
    rng = np.random.default_rng(int(alpha * 10))
    s = rng.normal(size=12)
    dp = rng.normal(size=12)
    ds = entmax_alpha_backward(s, dp, alpha)
    # ds = J^T dp; J is symmetric, checked through the full transpose product
    np.testing.assert_allclose(ds, _fd_jacobian(s, alpha).T @ dp, atol=1e-6)


def test_backward_alpha15_matches():
    rng = np.random.default_rng(5)
    s = rng.normal(size=(4, 33)) * 2
    dp = rng.normal(size=s.shape)
    allowed = rng.random(s.shape) > 0.2
    np.testing.assert_allclose(entmax_alpha_backward(s, dp, 1.5, allowed),
                               entmax15_backward(s, dp, allowed), atol=1e-12)


@pytest.mark.parametrize("alpha", [1.25, 1.75, 2.0])
def test_vjp_at_exact_p_is_the_gradient(alpha):
    # at the exact output: the finite-difference gradient of alpha-entmax
    rng = np.random.default_rng(int(alpha * 100) + 7)
    s = rng.normal(size=12)
    dp = rng.normal(size=12)
    p, _ = entmax_alpha_exact(s, alpha)
    ds = entmax_alpha_vjp(p, dp, alpha)[0]
    np.testing.assert_allclose(ds, _fd_jacobian(s, alpha).T @ dp, atol=1e-6)


def test_vjp_sparsemax_closed_form():
    # alpha = 2 (sparsemax): w is the support indicator, so ds = dp minus its
    # mean over the support, and zero off it; a row without support gets 0
    p = np.array([[0.75, 0.25, 0.0], [0.0, 0.0, 0.0]])
    dp = np.array([[1.0, -2.0, 5.0], [1.0, 2.0, 3.0]])
    np.testing.assert_allclose(entmax_alpha_vjp(p, dp, 2.0), [[1.5, -1.5, 0.0], [0.0, 0.0, 0.0]], atol=1e-15)


def test_rejects_alpha_outside():
    for a in (1.0, 0.5, 2.5):
        with pytest.raises(ValueError):
            entmax_alpha_exact(np.zeros(4), a)
