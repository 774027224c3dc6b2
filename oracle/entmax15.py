"""Plain float64 implementation of 1.5-entmax and 1.5-entmax attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and obvious on
purpose: one (batch, head) at a time, dense score matrices, numpy sort.

Notation follows "ADASPLASH -- ROBERTA Benchmark Result", section 2:
s is a row of scores, p = [(s - tau)/2]_+^2, g(tau) = sum_j p_j, tau the
unique root of g(tau) = 1.
"""

import numpy as np


# ---------------------------------------------------------------------------
# Allowed-key sets (masking)
# ---------------------------------------------------------------------------

def allowed_mask(L, key_mask_row=None, causal=False, window=0):
    """Boolean [L, L] matrix: entry (i, j) is True when query i may attend key j.

    Follows "ADASPLASH -- ROBERTA Benchmark Result", section 3 (padding mask,
    then causal tril for decoders, then the splash window for decoders), read
    as follows:

    * padding: key j is allowed only if key_mask_row[j] != 0 (padded keys are
      removed from the simplex rather than filled with a large negative value);
    * causal: j <= i;
    * window W > 0 (decoders only, so it requires causal): i - W < j <= i,
      i.e. W keys including the query itself.
    """
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    ok = np.ones((L, L), dtype=bool)
    if key_mask_row is not None:
        ok &= (np.asarray(key_mask_row) != 0)[None, :]
    if causal:
        ok &= j <= i
    if window > 0:
        if not causal:
            raise ValueError("the splash window is only defined for causal attention")
        ok &= j > i - window
    return ok


# ---------------------------------------------------------------------------
# 1.5-entmax on rows
# ---------------------------------------------------------------------------

def entmax15_exact(s, allowed=None):
    """Exact 1.5-entmax of each row of ``s`` over its allowed entries.

    Theorem 1 ("ADASPLASH -- ROBERTA Benchmark Result", section 2.2): the
    solution is p_j = ((s_j - tau)/2)^2 for s_j > tau and 0 otherwise, with
    tau the unique value where the p sum to 1.  On a support made of the k
    largest entries z_1 >= ... >= z_k this is sum_{i<=k} (z_i - tau)^2 = 4,
    i.e. (mean_k - tau)^2 = 4/k - var_k, and the root below the mean is
    tau_k = mean_k - sqrt(4/k - var_k).  The support is the largest k whose
    tau_k exists and lies below z_k (KKT conditions of the same theorem).

    Returns (p, tau).  Rows with no allowed entry get p = 0 and tau = +inf.
    """
    s = np.asarray(s, dtype=np.float64)
    squeeze = s.ndim == 1
    s = np.atleast_2d(s)
    R, N = s.shape
    if allowed is None:
        allowed = np.ones_like(s, dtype=bool)
    allowed = np.broadcast_to(np.atleast_2d(np.asarray(allowed, dtype=bool)), s.shape)
    if not np.all(np.isfinite(s[allowed])):
        raise ValueError("scores must be finite")

    n = allowed.sum(axis=1)
    z = np.where(allowed, s, -np.inf)
    z = -np.sort(-z, axis=1)                       # descending, disallowed last
    top = np.where(n > 0, z[:, 0], 0.0)
    k = np.arange(1, N + 1, dtype=np.float64)[None, :]
    in_row = k <= n[:, None]
    y = np.where(in_row, z - top[:, None], 0.0)    # shifted: largest is 0
    mean = np.cumsum(y, axis=1) / k
    var = np.maximum(np.cumsum(y * y, axis=1) / k - mean * mean, 0.0)
    delta = 4.0 / k - var
    tau_k = mean - np.sqrt(np.maximum(delta, 0.0))
    ok = in_row & (delta >= 0.0) & (y > tau_k)
    # largest admissible k (k = 1 is always admissible for a non-empty row)
    kstar = np.where(ok.any(axis=1), N - 1 - np.argmax(ok[:, ::-1], axis=1), -1)

    tau = np.full(R, np.inf)
    has = n > 0
    tau[has] = top[has] + tau_k[has, kstar[has]]

    above = allowed & (s > tau[:, None])
    p = np.where(above, ((s - tau[:, None]) / 2.0) ** 2, 0.0)

    # KKT consistency: the support found equals {j : s_j > tau}, up to
    # entries tied with tau to rounding (repeated score values, as low
    # precision inputs have, put whole tie groups at the boundary); those
    # carry p = ((s - tau)/2)^2 of the order of the rounding squared
    supp = above.sum(axis=1)
    bad = has & (supp != kstar + 1)
    if np.any(bad):
        scale = np.maximum(1.0, np.abs(np.where(has, top, 0.0)))
        near = np.abs(s - tau[:, None]) <= 1e-12 * scale[:, None]
        extra = above & ~near
        kept = extra.sum(axis=1)
        if np.any(kept[bad] > kstar[bad] + 1):
            raise AssertionError("support search inconsistent with KKT conditions")
    if squeeze:
        return p[0], tau[0]
    return p, tau


def entmax15_backward(s, dp, allowed=None):
    """Gradient of the scores from the gradient of p = entmax15(s), per row.

    Jacobian of "ADASPLASH -- ROBERTA Benchmark Result", section 2.4: with
    w = sqrt(p) (zero off the support), dp/ds = diag(w) - w w^T / sum(w), so
    ds = w * dp - w * (w . dp) / sum(w).  A row without an allowed entry has
    ds = 0.  Returns ds with the shape of s.
    """
    p, _ = entmax15_exact(s, allowed)
    p = np.atleast_2d(p)
    dp = np.atleast_2d(np.asarray(dp, dtype=np.float64))
    w = np.sqrt(p)
    den = w.sum(axis=1, keepdims=True)
    c = np.where(den > 0, (w * dp).sum(axis=1, keepdims=True) / np.where(den > 0, den, 1.0), 0.0)
    ds = w * (dp - c)
    return ds[0] if np.ndim(s) == 1 else ds


def entmax15_bisect(s, allowed=None, n_iter=25):
    """1.5-entmax by bisection on g(tau) = sum_j [(s_j - tau)/2]_+^2.

    Theorem 2 ("ADASPLASH -- ROBERTA Benchmark Result", section 2.3): g is
    strictly decreasing where positive, so bisection converges.  Bracket from
    "DistilBERT SST-2 with AdaSplash Attention", Mathematical Formulation 2:
    [max - 2, max - 2/sqrt(n)] with n the number of allowed entries.  Update
    rule: if g(mid) > 1 the root lies above mid (lo = mid), else hi = mid; the
    answer is the midpoint of the final bracket.  No renormalisation.

    Independent of ``entmax15_exact``: used by the tests to pin it.
    """
    s = np.asarray(s, dtype=np.float64)
    squeeze = s.ndim == 1
    s = np.atleast_2d(s)
    if allowed is None:
        allowed = np.ones_like(s, dtype=bool)
    allowed = np.broadcast_to(np.atleast_2d(np.asarray(allowed, dtype=bool)), s.shape)
    n = allowed.sum(axis=1)
    m = np.where(allowed, s, -np.inf).max(axis=1)
    has = n > 0
    m = np.where(has, m, 0.0)
    lo = m - 2.0
    hi = m - 2.0 / np.sqrt(np.maximum(n, 1))

    def g(t):
        d = np.where(allowed, np.maximum((s - t[:, None]) / 2.0, 0.0), 0.0)
        return (d * d).sum(axis=1)

    for _ in range(n_iter):
        mid = 0.5 * (lo + hi)
        up = g(mid) > 1.0
        lo = np.where(up, mid, lo)
        hi = np.where(up, hi, mid)
    tau = 0.5 * (lo + hi)
    tau = np.where(has, tau, np.inf)
    p = np.where(allowed & (s > tau[:, None]), ((s - tau[:, None]) / 2.0) ** 2, 0.0)
    if squeeze:
        return p[0], tau[0]
    return p, tau


def tsallis15_objective(p, s):
    """p.s + H_1.5(p), with H_1.5(p) = (4/3) sum (p - p^1.5).

    "ADASPLASH -- ROBERTA Benchmark Result", section 2.1 (H_alpha with
    alpha = 1.5, so 1/(alpha(alpha-1)) = 4/3); 1.5-entmax is its maximiser
    over the simplex.
    """
    p = np.asarray(p, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    return float(p @ s + (4.0 / 3.0) * np.sum(p - p ** 1.5))


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _as64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):            # torch tensor: exact upcast on the CPU
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _key_mask_row(key_mask, b):
    if key_mask is None:
        return None
    km = key_mask
    if hasattr(km, "detach"):
        km = km.detach().to("cpu").numpy()
    return np.asarray(km)[b]


def _head_list(B, H, heads):
    if heads is None:
        return [(b, h) for b in range(B) for h in range(H)]
    return [tuple(x) for x in heads]


def attention_forward(q, k, v, key_mask=None, causal=False, window=0,
                      heads=None, rows=None, return_probs=False):
    """1.5-entmax attention forward for the selected (b, h) heads.

    Scores s_ij = (q_i . k_j) / sqrt(d) ("ADASPLASH -- ROBERTA Benchmark
    Result", sections 3-4: logits = q k^T * d^-1/2; the model cards write /8
    for d = 64).  Row i takes 1.5-entmax over its allowed keys
    (``allowed_mask``), and O_i = sum_j A_ij V_j ("RoBERTa Base with AdaSplash
    Attention", Architecture Overview).

    Arguments: q [B, H, L, d], k, v [B, H_kv, L, d] (numpy or torch, any
    float dtype: upcast exactly to float64; H_kv divides H, and query head h
    reads key/value head h // (H / H_kv), the grouped-query repeat of K and V
    in "ADASPLASH -- ROBERTA Benchmark Result", section 3), key_mask [B, L]
    (nonzero = valid key) or None.  ``rows`` optionally restricts the query
    rows computed (same for every head).  Returns a dict with 'out'
    [nh, r, d], 'tau' [nh, r] and, when asked, 'probs' [nh, r, L]; 'heads'
    lists the (b, h) pairs in order.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, L, d = q.shape
    rep = H // k.shape[1]
    scale = 1.0 / np.sqrt(d)
    hl = _head_list(B, H, heads)
    r_idx = np.arange(L) if rows is None else np.asarray(rows)
    outs, taus, probs = [], [], []
    for (b, h) in hl:
        ok = allowed_mask(L, _key_mask_row(key_mask, b), causal, window)[r_idx]
        s = (q[b, h, r_idx] @ k[b, h // rep].T) * scale
        p, tau = entmax15_exact(s, ok)
        outs.append(p @ v[b, h // rep])
        taus.append(tau)
        if return_probs:
            probs.append(p)
    res = {"out": np.stack(outs), "tau": np.stack(taus), "heads": hl, "rows": r_idx}
    if return_probs:
        res["probs"] = np.stack(probs)
    return res


def attention_backward(q, k, v, dout, key_mask=None, causal=False, window=0,
                       heads=None, row_chunk=1024):
    """Gradients of 1.5-entmax attention w.r.t. q, k and v.

    Jacobian from "ADASPLASH -- ROBERTA Benchmark Result", section 2.4 (also
    "RoBERTa Base with AdaSplash Attention", Mathematical Formulation 2):
    for a row with p = entmax15(s) and incoming gradient g = dL/dp,
        dL/ds_j = sqrt(p_j) * (g_j - sum_k sqrt(p_k) g_k / sum_k sqrt(p_k)),
    which is zero off the support.  With O = A V: dL/dA = dO V^T, dV = A^T dO,
    and through s = q k^T / sqrt(d): dq = dS k / sqrt(d), dk = dS^T q / sqrt(d).

    Rows are processed in chunks of ``row_chunk`` to bound memory; the sums
    over rows for dk and dv are plain accumulations.  k and v may have
    H_kv heads (see ``attention_forward``).  Returns a dict with 'dq', 'dk',
    'dv' [nh, L, d] (dk, dv: the contribution of each query head), 'heads'
    and 'dk_kv', 'dv_kv' [B, H_kv, L, d]: the contributions summed over the
    query heads of each key/value head (the gradients of k and v when every
    head is selected).
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, H, L, d = q.shape
    Hkv = k.shape[1]
    rep = H // Hkv
    scale = 1.0 / np.sqrt(d)
    hl = _head_list(B, H, heads)
    dqs, dks, dvs = [], [], []
    dk_kv = np.zeros((B, Hkv, L, d))
    dv_kv = np.zeros((B, Hkv, L, d))
    for (b, h) in hl:
        kmr = _key_mask_row(key_mask, b)
        hk = h // rep
        dq = np.zeros((L, d))
        dk = np.zeros((L, d))
        dv = np.zeros((L, d))
        for r0 in range(0, L, row_chunk):
            r = np.arange(r0, min(L, r0 + row_chunk))
            ok = allowed_mask(L, kmr, causal, window)[r]
            s = (q[b, h, r] @ k[b, hk].T) * scale
            p, _ = entmax15_exact(s, ok)
            w = np.sqrt(p)                                  # sqrt(p), 0 off support
            gp = dout[b, h, r] @ v[b, hk].T                 # dL/dA
            den = w.sum(axis=1, keepdims=True)
            c = np.where(den > 0, (w * gp).sum(axis=1, keepdims=True) / np.where(den > 0, den, 1.0), 0.0)
            ds = w * (gp - c)
            dq[r] = (ds @ k[b, hk]) * scale
            dk += (ds.T @ q[b, h, r]) * scale
            dv += p.T @ dout[b, h, r]
        dqs.append(dq)
        dks.append(dk)
        dvs.append(dv)
        dk_kv[b, hk] += dk
        dv_kv[b, hk] += dv
    return {"dq": np.stack(dqs), "dk": np.stack(dks), "dv": np.stack(dvs), "heads": hl,
            "dk_kv": dk_kv, "dv_kv": dv_kv}


def attention_decode(q, k_cache, v_cache, seqlens, window=0, causal=True):
    """1.5-entmax attention for the newest queries of each sequence against a
    key/value cache (decode time for the causal decoders of "ADASPLASH --
    ROBERTA Benchmark Result", section 3, with the splash window of section
    7.1's decoder configuration).

    Arguments: q [B, H, d] (one new query per sequence) or [B, H, Lq, d];
    k_cache, v_cache [B, H_kv, S, d] (H_kv divides H, grouped-query repeat as
    in ``attention_forward``); seqlens [B]: the cache of sequence b holds
    n_b = seqlens[b] valid positions (clamped to [0, S]), the newest Lq of
    them the queries' own keys and values, so query i sits at position
    n_b - Lq + i (the queries are the last Lq positions of the sequence).
    Causality allows keys j <= that position; window W > 0 allows keys
    j > position - W only (W keys including the query's own).  With
    causal=False every one of the n_b cached keys is allowed to every query
    (query length below key length without a causal mask; window must be
    0).  Scores q . k_j / sqrt(d), 1.5-entmax over the allowed keys, O = A V.

    Returns (out, tau) shaped like q without / with its last axis; a query
    with no allowed key (its position below 0) gets O = 0 and tau = +inf.
    """
    q, k, v = _as64(q), _as64(k_cache), _as64(v_cache)
    single = q.ndim == 3
    if window > 0 and not causal:
        raise ValueError("the splash window is only defined for causal attention")
    if single:
        q = q[:, :, None, :]
    B, H, Lq, d = q.shape
    S = k.shape[2]
    rep = H // k.shape[1]
    sl = np.asarray(seqlens.detach().cpu().numpy() if hasattr(seqlens, "detach") else seqlens)
    out = np.zeros((B, H, Lq, d))
    tau = np.full((B, H, Lq), np.inf)
    for b in range(B):
        n = int(min(max(int(sl[b]), 0), S))
        for i in range(Lq):
            pos = n - Lq + i if causal else n - 1
            if pos < 0:
                continue
            lo = max(0, pos - window + 1) if window > 0 else 0
            for h in range(H):
                s = (k[b, h // rep, lo:pos + 1] @ q[b, h, i]) / np.sqrt(d)
                p, t = entmax15_exact(s)
                out[b, h, i] = p @ v[b, h // rep, lo:pos + 1]
                tau[b, h, i] = t
    if single:
        return out[:, :, 0], tau[:, :, 0]
    return out, tau


def attention_decode_backward(q, k_cache, v_cache, dout, seqlens, window=0, causal=True):
    """Gradients of ``attention_decode`` w.r.t. q, k_cache and v_cache.

    The same Jacobian as ``attention_backward`` ("ADASPLASH -- ROBERTA
    Benchmark Result", section 2.4): per query row with p = entmax15(s) over
    its allowed keys, w = sqrt(p), dp_j = dO . v_j, c = sum w dp / sum w,
    dS_j = w_j (dp_j - c); dq = dS K / sqrt(d), and every row adds
    dS_j q / sqrt(d) to dk_j and p_j dO to dv_j of its key/value head.
    Keys no query may attend (past n_b, or outside every window) get zero.

    Arguments as ``attention_decode`` plus dout shaped like q.  Returns
    (dq, dk, dv): dq like q, dk and dv like the caches, float64.
    """
    q, k, v, do = _as64(q), _as64(k_cache), _as64(v_cache), _as64(dout)
    single = q.ndim == 3
    if window > 0 and not causal:
        raise ValueError("the splash window is only defined for causal attention")
    if single:
        q, do = q[:, :, None, :], do[:, :, None, :]
    B, H, Lq, d = q.shape
    S = k.shape[2]
    rep = H // k.shape[1]
    sl = np.asarray(seqlens.detach().cpu().numpy() if hasattr(seqlens, "detach") else seqlens)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    sc = 1.0 / np.sqrt(d)
    for b in range(B):
        n = int(min(max(int(sl[b]), 0), S))
        for i in range(Lq):
            pos = n - Lq + i if causal else n - 1
            if pos < 0:
                continue
            lo = max(0, pos - window + 1) if window > 0 else 0
            for h in range(H):
                kh, vh = k[b, h // rep, lo:pos + 1], v[b, h // rep, lo:pos + 1]
                p, _ = entmax15_exact((kh @ q[b, h, i]) * sc)
                w = np.sqrt(p)
                dp = vh @ do[b, h, i]
                c = (w * dp).sum() / w.sum()
                ds = w * (dp - c)
                dq[b, h, i] = (ds @ kh) * sc
                dk[b, h // rep, lo:pos + 1] += np.outer(ds, q[b, h, i]) * sc
                dv[b, h // rep, lo:pos + 1] += np.outer(p, do[b, h, i])
    if single:
        return dq[:, :, 0], dk, dv
    return dq, dk, dv
