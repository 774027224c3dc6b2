"""GPU parity on seeded random shapes: batch, heads, length (short, long and
stream paths), head dimension, dtype, causal mask and window, padding and
score scale drawn from a fixed generator, forward checked on every row of
one head per case, backward on the short cases.  Same bar as
test_parity_gpu.py.  Cases of the first batch share the head count of K
and V with Q; the second batch draws grouped-query heads too."""

import numpy as np
import pytest
import torch

from entmax_amd.workloads import random_inputs
from tests.parity_util import check_backward, check_forward

pytestmark = pytest.mark.gpu


def _cases(n=20, seed=2024, bands=3, gains=(0.3, 1.0, 2.0), gqa=False):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        band = i % bands
        L = int(rng.integers(1, 129) if band == 0 else rng.integers(129, 1025) if band == 1
                else rng.integers(1025, 2500) if band == 2 else rng.integers(2049, 3200))
        causal = bool(rng.random() < 0.5)
        window = int(rng.choice([0, 1, 7, 32, 100])) if causal else 0
        out.append(dict(B=int(rng.integers(1, 4)), H=int(rng.integers(1, 4)), L=L, d=int(rng.choice([64, 128])),
                        dtype=str(rng.choice(["f32", "bf16"])), causal=causal, window=window,
                        pad=str(rng.choice(["none", "right", "scattered"])), gain=float(rng.choice(gains)),
                        hkv_div=int(rng.choice([1, 2, 4])) if gqa else 1, seed=seed + i))
        # the float32 bar (1e-5 absolute) is the precision of float32 work on
        # scores of order one, as in the pages' workloads: a score computed
        # from d products carries a rounding error that grows with its size
        # (about 1e-5 at |s| ~ 16), so float32 cases keep scores of order one
        if out[-1]["dtype"] == "f32":
            out[-1]["gain"] = min(out[-1]["gain"], 1.0)
    return out


# second batch: grouped-query heads, the stream path (spans above 2048) and
# a wider range of score scales
CASES = _cases() + _cases(n=24, seed=7777, bands=4, gains=(0.1, 0.3, 1.0, 2.0, 4.0), gqa=True)


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_random_shape(case):
    c = case
    rng = np.random.default_rng(c["seed"])
    kw = {}
    if c["pad"] == "right":
        kw["key_lengths"] = [int(x) for x in rng.integers(0, c["L"] + 1, size=c["B"])]
    elif c["pad"] == "scattered":
        kw["key_mask_density"] = 0.7
    H = c["H"] * c["hkv_div"]
    inp = random_inputs(c["B"], H, c["L"], c["d"], c["dtype"], seed=c["seed"], qk_gain=c["gain"], **kw)
    hkv = H // c["hkv_div"]
    for name in ("k", "v"):
        inp[name] = inp[name][:, :hkv].contiguous()
    inp["causal"], inp["window"] = c["causal"], c["window"]
    label = (f"random B{c['B']} H{H}/{hkv} L{c['L']} d{c['d']} {c['dtype']} causal={c['causal']} "
             f"W{c['window']} pad={c['pad']} gain={c['gain']}")
    head = [(c["B"] - 1, H - 1)]
    check_forward(inp, heads=head, label=label)
    if c["L"] <= 300:
        # grouped K, V: their gradients sum over every query head of the group
        check_backward(inp, heads=head if hkv == H else None, label=label)


def _decode_cases(n=16, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        S = int(rng.choice([int(rng.integers(1, 257)), int(rng.integers(257, 5000))]))
        causal = bool(rng.random() < 0.75)
        dtype = str(rng.choice(["f32", "bf16"]))
        out.append(dict(B=int(rng.integers(1, 5)), Hkv=int(rng.integers(1, 4)), G=int(rng.choice([1, 2, 4, 8, 20])),
                        Lq=int(rng.choice([1, 1, 3, 16, 40])), S=S, d=int(rng.choice([64, 128])), dtype=dtype,
                        causal=causal, window=int(rng.choice([0, 32, 100])) if causal else 0,
                        gain=float(rng.choice([0.3, 1.0] if dtype == "f32" else [0.3, 1.0, 2.0])), seed=seed + i))
    return out


DEC_CASES = _decode_cases()


@pytest.mark.parametrize("case", DEC_CASES, ids=[f"d{i}" for i in range(len(DEC_CASES))])
def test_random_decode(case):
    from entmax_amd import entmax_attn_decode
    from oracle import attention_decode
    from tests.parity_util import TOL, log
    c = case
    rng = np.random.default_rng(c["seed"])
    H = c["Hkv"] * c["G"]
    Lq = min(c["Lq"], c["S"])
    gen = torch.Generator().manual_seed(c["seed"])
    dt = torch.float32 if c["dtype"] == "f32" else torch.bfloat16
    q = (torch.randn((c["B"], H, Lq, c["d"]), generator=gen) * c["gain"]).to(dt)
    k = (torch.randn((c["B"], c["Hkv"], c["S"], c["d"]), generator=gen) * c["gain"]).to(dt)
    v = torch.randn((c["B"], c["Hkv"], c["S"], c["d"]), generator=gen).to(dt)
    sl = torch.tensor([int(x) for x in rng.integers(0, c["S"] + 1, size=c["B"])], dtype=torch.int32)
    log(f"[decode] random {c} seqlens {sl.tolist()}")
    out, tau = entmax_attn_decode(q.cuda(), k.cuda(), v.cuda(), sl.cuda(), c["window"], causal=c["causal"])
    torch.cuda.synchronize()
    ref_o, ref_t = attention_decode(q, k, v, sl.numpy(), c["window"], causal=c["causal"])
    t = tau.cpu().numpy()
    assert np.array_equal(np.isinf(t), np.isinf(ref_t))
    fin = np.isfinite(ref_t)
    err_o = float(np.abs(out.cpu().numpy() - ref_o).max())
    err_t = float(np.abs(t[fin] - ref_t[fin]).max()) if fin.any() else 0.0
    log(f"[decode]   max err O={err_o:.3g} tau={err_t:.3g}")
    assert err_o <= TOL[c["dtype"]] and err_t <= TOL[c["dtype"]]


def _rows_cases(n=12, seed=99):
    rng = np.random.default_rng(seed)
    return [dict(R=int(rng.integers(1, 3000)), L=4 * int(rng.integers(1, 2500)), alpha=float(rng.choice([1.5, 1.2, 1.8, 2.0])),
                 dtype=str(rng.choice(["f32", "bf16"])), gain=float(rng.choice([0.3, 1.0, 3.0])),
                 mask=bool(rng.random() < 0.5), seed=seed + i) for i in range(n)]


ROW_CASES = _rows_cases()


@pytest.mark.parametrize("case", ROW_CASES, ids=[f"r{i}" for i in range(len(ROW_CASES))])
def test_random_rows(case):
    # row-wise alpha-entmax and its backward on sampled rows
    from entmax_amd import entmax_bisect_rows, entmax_bisect_rows_bwd
    from oracle import entmax_alpha_backward, entmax_alpha_exact
    from tests.parity_util import TOL, log
    c = case
    gen = torch.Generator().manual_seed(c["seed"])
    dt = torch.float32 if c["dtype"] == "f32" else torch.bfloat16
    s = (torch.randn((c["R"], c["L"]), generator=gen) * c["gain"]).to(dt)
    mask = (torch.rand((c["R"], c["L"]), generator=gen) > 0.3).to(torch.uint8) if c["mask"] else None
    dp = torch.randn((c["R"], c["L"]), generator=gen)
    log(f"[rows] random {c}")
    p, tau = entmax_bisect_rows(s.cuda(), c["alpha"], None if mask is None else mask.cuda())
    ds = entmax_bisect_rows_bwd(p, dp.cuda(), c["alpha"])
    torch.cuda.synchronize()
    rows = np.random.default_rng(c["seed"]).choice(c["R"], min(c["R"], 24), replace=False)
    ok = None if mask is None else mask.numpy()[rows] != 0
    s64 = s[rows].to(torch.float64).numpy()
    p_ref, t_ref = entmax_alpha_exact(s64, c["alpha"], ok)
    tol = TOL[c["dtype"]]
    assert float(np.abs(p.cpu().numpy()[rows] - p_ref).max()) <= tol
    fin = np.isfinite(t_ref)
    assert float(np.abs(tau.cpu().numpy()[rows][fin] - t_ref[fin]).max()) <= tol
    dp64 = dp[rows].double().numpy()
    ref = entmax_alpha_backward(s64, dp64, c["alpha"], ok)
    # the backward entry point on the oracle's p (rounded to float32): its
    # own parity, for every alpha
    ds_o = entmax_bisect_rows_bwd(torch.from_numpy(p_ref).float().cuda(), dp[rows].contiguous().cuda(), c["alpha"])
    err = float(np.abs(ds_o.cpu().numpy() - ref).max()) / max(1.0, float(np.abs(ref).max()))
    log(f"[rows]   scaled bwd err on the oracle's p {err:.3g}")
    assert err <= TOL["f32"]
    # the chain forward -> backward.  (1) Every row against the exact
    # backward taken at the kernel's own output p: the backward's arithmetic
    # given the forward.  (2) Against the exact backward: every row for
    # alpha <= 1.5, where w = p^(2 - alpha) is Lipschitz in tau; above 1.5
    # the slope of w is unbounded at the support boundary, so rows with an
    # allowed entry within the band where the measured tau error would move
    # w by more than 1e-6 are exempt (chain_rows_ok), and the rest compared.
    from oracle import entmax_alpha_vjp
    from tests.parity_util import chain_rows_ok
    dsr = ds.cpu().numpy()[rows]
    tg = tau.cpu().numpy()[rows].astype(np.float64)
    ref_at = entmax_alpha_vjp(p.cpu().numpy()[rows], dp64, c["alpha"])
    err = float(np.abs(dsr - ref_at).max()) / max(1.0, float(np.abs(ref_at).max()))
    log(f"[rows]   scaled bwd err after the kernel's forward, at its p {err:.3g}")
    assert err <= TOL["f32"]
    keep, band = chain_rows_ok(s64, tg, t_ref, c["alpha"], ok)
    if keep.any():
        err = float(np.abs(dsr[keep] - ref[keep]).max()) / max(1.0, float(np.abs(ref[keep]).max()))
        log(f"[rows]   scaled bwd err after the kernel's forward {err:.3g} ({int(keep.sum())} of {len(keep)} rows; "
            f"band up to {float(band.max()):.2g})")
        assert err <= TOL["f32"]


def _bwd_cases(n=10, seed=555):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = str(rng.choice(["f32", "bf16"]))
        causal = bool(rng.random() < 0.5)
        out.append(dict(B=1, H=int(rng.integers(1, 3)), L=int(rng.integers(301, 2600)), d=int(rng.choice([64, 128])),
                        dtype=dtype, causal=causal, window=int(rng.choice([0, 32])) if causal else 0,
                        gain=float(rng.choice([0.3, 1.0] if dtype == "f32" else [0.3, 1.0, 2.0])), seed=seed + i))
    return out


BWD_CASES = _bwd_cases()


@pytest.mark.parametrize("case", BWD_CASES, ids=[f"b{i}" for i in range(len(BWD_CASES))])
def test_random_backward_long(case):
    # the backward on spans the short cases above do not reach (dense and
    # sparse supports, candidate lists that overflow)
    c = case
    inp = random_inputs(c["B"], c["H"], c["L"], c["d"], c["dtype"], seed=c["seed"], qk_gain=c["gain"])
    inp["causal"], inp["window"] = c["causal"], c["window"]
    check_backward(inp, heads=[(0, c["H"] - 1)], label=f"random bwd {c}")
