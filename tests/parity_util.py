"""Helpers for GPU-vs-oracle parity checks (test code only)."""

import math
import sys

import numpy as np
import torch

from oracle import allowed_mask, attention_backward, attention_forward

TOL = {"f32": 1e-5, "bf16": 2e-3}     # absolute, on A, O and tau
NEAR_TAU = 1e-6                       # zero-pattern exemption band around tau


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dtype_name(t):
    return "f32" if t.dtype == torch.float32 else "bf16"


def to_gpu(inp):
    out = dict(inp)
    for k in ("q", "k", "v", "dout", "key_mask"):
        if out.get(k) is not None:
            out[k] = out[k].cuda()
    return out


def scores64(q, k, b, h, rows):
    # k may have fewer (grouped) heads: query head h reads k head h // (H / H_kv)
    q64 = q[b, h].to(torch.float64).cpu().numpy()
    k64 = k[b, h // (q.shape[1] // k.shape[1])].to(torch.float64).cpu().numpy()
    return (q64[rows] @ k64.T) / math.sqrt(q.shape[-1])


def head_probs(q, k, tau, km, causal, window, b, h):
    """Dense A of one (b, h) from the GPU's probs export ([L, L] numpy)."""
    from entmax_amd import entmax_attn_probs
    hk = h // (q.shape[1] // k.shape[1])
    pr = entmax_attn_probs(q[b:b + 1, h:h + 1].contiguous(), k[b:b + 1, hk:hk + 1].contiguous(),
                           tau[b:b + 1, h:h + 1].contiguous(), None if km is None else km[b:b + 1].contiguous(),
                           causal, window)
    return pr[0, 0].cpu().numpy()


def check_forward(inp, heads=None, rows=None, check_probs=True, label="", band=NEAR_TAU):
    """Run the HIP forward on `inp` (CPU tensors) and compare with the oracle
    on the selected heads / rows.  Returns a dict of max errors.

    With check_probs, A (from the probs export, one head at a time) is
    compared entry by entry and the exact-zero pattern must agree except for
    entries within ``band`` of tau (the oracle's)."""
    from entmax_amd import entmax_attn_fwd, entmax_attn_probs
    g = to_gpu(inp)
    q, k, v, km = g["q"], g["k"], g["v"], g["key_mask"]
    causal, window = bool(inp["causal"]), int(inp["window"])
    B, H, L, d = q.shape
    tol = TOL[dtype_name(q)]
    log(f"[parity] fwd {label} B{B} H{H} L{L} d{d} {dtype_name(q)} causal={causal} window={window}")
    out, tau = entmax_attn_fwd(q, k, v, km, causal, window)
    torch.cuda.synchronize()
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    r_idx = np.arange(L) if rows is None else np.asarray(rows)
    ref = attention_forward(inp["q"], inp["k"], inp["v"], inp["key_mask"], causal, window,
                            heads=heads, rows=r_idx, return_probs=check_probs)
    out_c = out.cpu().numpy()
    tau_c = tau.cpu().numpy()
    errs = {"out": 0.0, "tau": 0.0, "probs": 0.0, "pattern_bad": 0}
    km_np = None if inp["key_mask"] is None else inp["key_mask"].numpy()
    for n, (b, h) in enumerate(heads):
        o_gpu = out_c[b, h][r_idx]
        t_gpu = tau_c[b, h][r_idx]
        t_ref = ref["tau"][n]
        inf_ref = np.isinf(t_ref)
        assert np.array_equal(np.isinf(t_gpu), inf_ref), f"empty-row pattern differs at head {(b, h)}"
        errs["out"] = max(errs["out"], float(np.abs(o_gpu - ref["out"][n]).max()))
        if (~inf_ref).any():
            errs["tau"] = max(errs["tau"], float(np.abs(t_gpu[~inf_ref] - t_ref[~inf_ref]).max()))
        if check_probs:
            a_gpu = head_probs(q, k, tau, km, causal, window, b, h)[r_idx]
            a_ref = ref["probs"][n]
            errs["probs"] = max(errs["probs"], float(np.abs(a_gpu - a_ref).max()))
            s = scores64(inp["q"], inp["k"], b, h, r_idx)
            ok = allowed_mask(L, None if km_np is None else km_np[b], causal, window)[r_idx]
            dist = np.abs(s - t_ref[:, None])
            differ = ((a_gpu == 0) != (a_ref == 0)) & ok
            errs["pattern_bad"] += int((differ & (dist > band)).sum())
            errs["pattern_flips"] = errs.get("pattern_flips", 0) + int(differ.sum())
            if differ.any():
                errs["flip_max_dist"] = max(errs.get("flip_max_dist", 0.0), float(dist[differ].max()))
            errs["support"] = errs.get("support", 0) + int((a_ref > 0).sum())
            assert not np.any((a_gpu != 0) & ~ok), "nonzero weight on a disallowed key"
    log(f"[parity]   max err out={errs['out']:.3g} tau={errs['tau']:.3g} probs={errs['probs']:.3g} "
        f"pattern_bad={errs['pattern_bad']} (band {band:.3g}; flips {errs.get('pattern_flips', 0)}, farthest "
        f"{errs.get('flip_max_dist', 0.0):.3g} from tau; support {errs.get('support', 0)}) (tol {tol})")
    assert errs["out"] <= tol, errs
    assert errs["tau"] <= tol, errs
    assert errs["probs"] <= tol, errs
    assert errs["pattern_bad"] == 0, errs
    return errs, out, tau


def check_backward(inp, heads=None, label="", tau=None, saved=False):
    """With saved: the forward keeps the support (entmax_attn_fwd_save) and
    the backward reads it (entmax_attn_bwd_saved)."""
    from entmax_amd import entmax_attn_bwd, entmax_attn_bwd_saved, entmax_attn_fwd, entmax_attn_fwd_save
    g = to_gpu(inp)
    q, k, v, do, km = g["q"], g["k"], g["v"], g["dout"], g["key_mask"]
    causal, window = bool(inp["causal"]), int(inp["window"])
    B, H, L, d = q.shape
    tol = TOL[dtype_name(q)]
    log(f"[parity] bwd {label} B{B} H{H} L{L} d{d} {dtype_name(q)} causal={causal} window={window} saved={saved}")
    if saved:
        _, tau, sv = entmax_attn_fwd_save(q, k, v, km, causal, window)
        dq, dk, dv = entmax_attn_bwd_saved(q, k, v, tau, do, sv, km, causal, window)
    else:
        if tau is None:
            _, tau = entmax_attn_fwd(q, k, v, km, causal, window)
        dq, dk, dv = entmax_attn_bwd(q, k, v, tau, do, km, causal, window)
    torch.cuda.synchronize()
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["dout"], inp["key_mask"], causal, window, heads=heads)
    grouped = k.shape[1] != H
    assert not grouped or len(heads) == B * H, "grouped k, v: every head is needed for their gradients"
    errs = {}
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        got_c = got.cpu().numpy()
        worst = 0.0
        if grouped and name != "dq":
            # dk, dv of a key/value head: the sum over its query heads
            r = ref[name + "_kv"]
            worst = float(np.abs(got_c - r).max()) / max(1.0, float(np.abs(r).max()))
        else:
            for n, (b, h) in enumerate(heads):
                r = ref[name][n]
                scale = max(1.0, float(np.abs(r).max()))
                worst = max(worst, float(np.abs(got_c[b, h] - r).max()) / scale)
        errs[name] = worst
    log(f"[parity]   max scaled err dq={errs['dq']:.3g} dk={errs['dk']:.3g} dv={errs['dv']:.3g} (tol {tol})")
    for name in ("dq", "dk", "dv"):
        assert errs[name] <= tol, errs
    return errs


def chain_rows_ok(s64, tau_gpu, tau_ref, alpha, ok=None, slope_err=1e-6):
    """Rows whose alpha-entmax backward is well conditioned in tau at the
    forward's error: no allowed entry so close to the exact tau that the
    weight w = p^(2 - alpha) = [(alpha - 1)(s - tau)]^k, k = (2 - alpha)/(alpha - 1),
    moves by more than ``slope_err`` under that row's tau error.  For
    alpha <= 1.5 (k >= 1) w is Lipschitz and every row qualifies; for
    1.5 < alpha < 2 the band is where k (alpha - 1)^k delta^(k - 1) eps
    exceeds slope_err; at alpha = 2 (w an indicator) it is twice the error;
    never below 1e-6 max(1, |tau|), the float32 resolution of the scores."""
    s64 = np.atleast_2d(s64)
    tg = np.asarray(tau_gpu, np.float64)
    tr = np.asarray(tau_ref, np.float64)
    fin = np.isfinite(tr)
    # rows with no allowed entry carry tau = +inf on both sides: no error there
    eps = np.where(fin, np.abs(np.where(fin, tg, 0.0) - np.where(fin, tr, 0.0)), 0.0)
    if alpha <= 1.5:
        return np.ones(s64.shape[0], bool), np.zeros(s64.shape[0])
    k = (2.0 - alpha) / (alpha - 1.0)
    if k == 0.0:
        band = 2.0 * eps
    else:
        with np.errstate(divide="ignore"):
            band = np.where(eps > 0, (slope_err / (k * (alpha - 1.0) ** k * np.maximum(eps, 1e-300))) ** (1.0 / (k - 1.0)), 0.0)
    # and at least the float32 resolution of the scores near tau, where the
    # two sides may round an entry to opposite sides of it
    band = np.maximum(np.maximum(band, 2.0 * eps), 1e-6 * np.maximum(1.0, np.abs(np.where(fin, tau_ref, 0.0))))
    allowed = np.ones_like(s64, bool) if ok is None else np.atleast_2d(ok)
    dist = np.abs(s64 - np.where(fin, tau_ref, 0.0)[:, None])
    near = ((dist < band[:, None]) & allowed).any(axis=1)
    return fin & ~near | ~fin, band
