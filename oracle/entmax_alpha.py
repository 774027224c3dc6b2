"""Plain float64 alpha-entmax on rows, for alpha in (1, 2].

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation follows "ADASPLASH -- ROBERTA Benchmark Result": section 2.1 defines
alpha-entmax as the maximiser of p.s + H_alpha(p) over the simplex, with the
Tsallis entropy H_alpha(p) = sum_j (p_j - p_j^alpha) / (alpha (alpha - 1));
the entmax_bisect routine of section 4 solves
sum_j [(alpha - 1) s_j - tau']_+^(1/(alpha - 1)) = 1.  Here the threshold is
kept in score units, tau = tau' / (alpha - 1), so that

    p_j = [(alpha - 1)(s_j - tau)]_+^(1/(alpha - 1)),   sum_j p_j = 1,

which for alpha = 1.5 is p_j = [(s_j - tau)/2]_+^2 (section 2.2, Theorem 1).
"""

import numpy as np
from scipy.optimize import brentq


def _rows(s, allowed):
    s = np.asarray(s, dtype=np.float64)
    squeeze = s.ndim == 1
    s = np.atleast_2d(s)
    if allowed is None:
        allowed = np.ones_like(s, dtype=bool)
    allowed = np.broadcast_to(np.atleast_2d(np.asarray(allowed, dtype=bool)), s.shape)
    return s, allowed, squeeze


def _check_alpha(alpha):
    if not (1.0 < alpha <= 2.0):
        raise ValueError(f"alpha = {alpha} outside (1, 2]")


def _probs(s_row, tau, alpha):
    """p_j = [(alpha - 1)(s_j - tau)]_+^(1/(alpha - 1)) for one row."""
    return np.maximum((alpha - 1.0) * (s_row - tau), 0.0) ** (1.0 / (alpha - 1.0))


def entmax_alpha_exact(s, alpha, allowed=None):
    """alpha-entmax of each row of ``s`` over its allowed entries, tau to
    float64 precision.

    The threshold is the root of g(tau) = sum_j p_j(tau) - 1 over the allowed
    entries.  g is continuous and strictly decreasing up to the row maximum m
    (the argument of section 2.3, Theorem 2, holds for any alpha > 1), with
    g(m) = -1 and g(m - 2/(alpha - 1)) > 0 (the maximum alone contributes
    2^(1/(alpha - 1)) > 1 there), so the root lies in that bracket; a library
    root finder (Brent's method) locates it to rounding.

    Returns (p, tau).  Rows with no allowed entry get p = 0 and tau = +inf.
    """
    _check_alpha(alpha)
    s, allowed, squeeze = _rows(s, allowed)
    if not np.all(np.isfinite(s[allowed])):
        raise ValueError("scores must be finite")
    R = s.shape[0]
    p = np.zeros_like(s)
    tau = np.full(R, np.inf)
    for r in range(R):
        z = s[r, allowed[r]]
        if z.size == 0:
            continue
        m = z.max()
        lo, hi = m - 2.0 / (alpha - 1.0), m

        def g(t):
            return _probs(z, t, alpha).sum() - 1.0

        t = brentq(g, lo, hi, xtol=1e-15 * max(1.0, abs(m)), rtol=1e-15, maxiter=500)
        tau[r] = t
        p[r] = np.where(allowed[r], _probs(s[r], t, alpha), 0.0)
    if squeeze:
        return p[0], tau[0]
    return p, tau


def entmax_alpha_bisect(s, alpha, allowed=None, n_iter=25):
    """alpha-entmax by bisection, in the order of the entmax_bisect routine of
    "ADASPLASH -- ROBERTA Benchmark Result", section 4: shift by the row
    maximum m and scale by alpha - 1, x_j = (alpha - 1)(s_j - m); bisect
    t on sum_j [x_j - t]_+^(1/(alpha - 1)) = 1 (sum > 1 moves the lower end,
    else the upper end); the answer is the midpoint of the final bracket.

    Bracket: [-1, -n^(1 - alpha)] with n the number of allowed entries (the
    maximum alone gives 1 at -1; at -n^(1-alpha) each of the n terms is at
    most 1/n).  For alpha = 1.5 this is the bracket [max - 2, max - 2/sqrt(n)]
    of "DistilBERT SST-2 with AdaSplash Attention", Mathematical Formulation
    2, in score units.  No renormalisation of p.  tau = m + t/(alpha - 1).
    """
    _check_alpha(alpha)
    s, allowed, squeeze = _rows(s, allowed)
    am1 = alpha - 1.0
    n = allowed.sum(axis=1)
    has = n > 0
    m = np.where(has, np.where(allowed, s, -np.inf).max(axis=1), 0.0)
    x = np.where(allowed, am1 * (s - m[:, None]), -np.inf)
    lo = np.full(s.shape[0], -1.0)
    hi = -np.maximum(n, 1).astype(np.float64) ** (1.0 - alpha)

    def total(t):
        return (np.maximum(x - t[:, None], 0.0) ** (1.0 / am1)).sum(axis=1)

    for _ in range(n_iter):
        mid = 0.5 * (lo + hi)
        up = total(mid) > 1.0
        lo = np.where(up, mid, lo)
        hi = np.where(up, hi, mid)
    t = 0.5 * (lo + hi)
    p = np.where(has[:, None], np.maximum(x - t[:, None], 0.0) ** (1.0 / am1), 0.0)
    tau = np.where(has, m + t / am1, np.inf)
    if squeeze:
        return p[0], tau[0]
    return p, tau


def entmax_alpha_backward(s, dp, alpha, allowed=None):
    """Gradient of the scores from the gradient of p = alpha-entmax(s), per row.

    On the support, p_j^(alpha - 1) = (alpha - 1)(s_j - tau) ("ADASPLASH --
    ROBERTA Benchmark Result", section 2.2 proof, stationarity for general
    alpha); differentiating under sum p = 1 gives dp/ds = diag(w) -
    w w^T / sum(w) with w = p^(2 - alpha) (zero off the support), which is
    section 2.4's Jacobian (w = sqrt(p)) at alpha = 1.5.  So
    ds = w * dp - w * (w . dp) / sum(w).  A row without an allowed entry has
    ds = 0.
    """
    p, _ = entmax_alpha_exact(s, alpha, allowed)
    p = np.atleast_2d(p)
    dp = np.atleast_2d(np.asarray(dp, dtype=np.float64))
    w = np.where(p > 0, p ** (2.0 - alpha), 0.0)
    den = w.sum(axis=1, keepdims=True)
    c = np.where(den > 0, (w * dp).sum(axis=1, keepdims=True) / np.where(den > 0, den, 1.0), 0.0)
    ds = w * (dp - c)
    return ds[0] if np.ndim(s) == 1 else ds


def entmax_alpha_vjp(p, dp, alpha):
    """The backward of entmax_alpha_backward taken at a given output p (each
    row a point of the simplex): w = p^(2 - alpha) on the support p > 0 (zero
    off it) and ds = w * dp - w * (w . dp) / sum(w) (section 2.4's Jacobian in
    the general-alpha form of section 2.2's stationarity).  At the exact p it
    is entmax_alpha_backward; at the p of another solve it is the gradient
    that solve's output leads to, which separates the backward's own
    arithmetic from the conditioning of w in tau (for alpha > 1.5 the slope
    of w is unbounded at the support boundary, and at alpha = 2 w is the
    support indicator).  Rows with no support get ds = 0.
    """
    _check_alpha(alpha)
    p = np.atleast_2d(np.asarray(p, dtype=np.float64))
    dp = np.atleast_2d(np.asarray(dp, dtype=np.float64))
    w = np.where(p > 0, np.where(p > 0, p, 1.0) ** (2.0 - alpha), 0.0)
    den = w.sum(axis=1, keepdims=True)
    c = np.where(den > 0, (w * dp).sum(axis=1, keepdims=True) / np.where(den > 0, den, 1.0), 0.0)
    return w * (dp - c)


def tsallis_objective(p, s, alpha):
    """p.s + H_alpha(p), H_alpha(p) = sum (p - p^alpha) / (alpha (alpha - 1))
    ("ADASPLASH -- ROBERTA Benchmark Result", section 2.1); alpha-entmax is
    its maximiser over the simplex."""
    p = np.asarray(p, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    return float(p @ s + np.sum(p - p ** alpha) / (alpha * (alpha - 1.0)))
