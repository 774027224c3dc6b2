"""GPU parity of decode-time attention (entmax_attn_decode through the C ABI)
against the float64 oracle ``attention_decode``: absolute error <= 1e-5
(float32 inputs) or 2e-3 (bfloat16 inputs) on O and tau, tau = +inf exactly
for empty caches."""

import numpy as np
import pytest
import torch

from oracle import attention_decode
from tests.parity_util import TOL, log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(B, H, Hkv, S, d, dtype, gain, seed, seqlens):
    gen = torch.Generator().manual_seed(seed)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = (torch.randn((B, H, d), generator=gen) * gain).to(dt)
    k = torch.randn((B, Hkv, S, d), generator=gen).to(dt)
    v = torch.randn((B, Hkv, S, d), generator=gen).to(dt)
    return q, k, v, torch.tensor(seqlens, dtype=torch.int32)


def _check(q, k, v, sl, window, dtype, out, tau, causal=True):
    ref_o, ref_t = attention_decode(q, k, v, sl.numpy(), window, causal=causal)
    o, t = out.cpu().numpy(), tau.cpu().numpy()
    assert np.array_equal(np.isinf(t), np.isinf(ref_t))
    fin = np.isfinite(ref_t)
    err_o = float(np.abs(o - ref_o).max())
    err_t = float(np.abs(t[fin] - ref_t[fin]).max()) if fin.any() else 0.0
    log(f"[decode]   max err O={err_o:.3g} tau={err_t:.3g}")
    assert err_o <= TOL[dtype] and err_t <= TOL[dtype]


CASES = [
    # (dtype, d, H, Hkv, S, window, gain)
    ("f32", 64, 4, 4, 40, 0, 1.0),
    ("f32", 64, 4, 4, 40, 32, 1.0),
    ("f32", 128, 8, 2, 300, 0, 2.0),
    ("f32", 64, 20, 1, 1100, 0, 1.0),
    ("f32", 128, 4, 4, 1100, 32, 2.0),
    ("bf16", 64, 4, 4, 40, 32, 1.0),
    ("bf16", 64, 12, 12, 300, 0, 1.0),
    ("bf16", 128, 8, 2, 1100, 0, 2.0),
    ("bf16", 64, 20, 1, 600, 32, 1.0),
    ("bf16", 128, 32, 8, 2100, 0, 2.0),
    ("bf16", 64, 6, 3, 513, 300, 1.0),
]


@pytest.mark.parametrize("dtype,d,H,Hkv,S,window,gain", CASES)
def test_decode_matches_oracle(dtype, d, H, Hkv, S, window, gain):
    from entmax_amd import entmax_attn_decode
    rng = np.random.default_rng(S + d + H)
    seqlens = [S, 1, int(rng.integers(2, S)), 0, min(S, 33)]
    q, k, v, sl = _inputs(5, H, Hkv, S, d, dtype, gain, seed=S * 7 + H, seqlens=seqlens)
    log(f"[decode] {dtype} d{d} H{H} Hkv{Hkv} S{S} W{window} seqlens {seqlens}")
    out, tau = entmax_attn_decode(q.cuda(), k.cuda(), v.cuda(), sl.cuda(), window)
    torch.cuda.synchronize()
    _check(q, k, v, sl, window, dtype, out, tau)


def test_decode_long_cache():
    # the long-context shape at decode time: 8192 cached keys, grouped queries
    from entmax_amd import entmax_attn_decode
    q, k, v, sl = _inputs(2, 32, 8, 8192, 128, "bf16", 2.0, seed=5, seqlens=[8192, 5000])
    log("[decode] bf16 d128 H32 Hkv8 S8192 W0")
    out, tau = entmax_attn_decode(q.cuda(), k.cuda(), v.cuda(), sl.cuda(), 0)
    torch.cuda.synchronize()
    _check(q, k, v, sl, 0, "bf16", out, tau)


def test_decode_very_long_cache():
    # 2^20 cached keys: 4096 chunks per row, and a row solve of more entries
    # than the registers of a workgroup hold (streamed at every step)
    from entmax_amd import entmax_attn_decode
    S = 1 << 20
    q, k, v, sl = _inputs(1, 2, 1, S, 64, "bf16", 1.0, seed=20, seqlens=[S])
    log("[decode] bf16 d64 H2 Hkv1 S2^20 W0")
    out, tau = entmax_attn_decode(q.cuda(), k.cuda(), v.cuda(), sl.cuda(), 0)
    torch.cuda.synchronize()
    _check(q, k, v, sl, 0, "bf16", out, tau)


def test_decode_reuses_workspace():
    # a second, smaller call on the same workspace sees nothing of the first
    from entmax_amd import decode_workspace_bytes, entmax_attn_decode
    ws = torch.empty((decode_workspace_bytes(3, 8, 4, 900, 64, 0, 1),), dtype=torch.uint8, device="cuda")
    for S, seqlens in ((900, [900, 700, 3]), (500, [10, 499, 0])):
        q, k, v, sl = _inputs(3, 8, 4, S, 64, "bf16", 1.0, seed=S, seqlens=seqlens)
        log(f"[decode] workspace reuse S{S} seqlens {seqlens}")
        out, tau = entmax_attn_decode(q.cuda(), k.cuda(), v.cuda(), sl.cuda(), 0, workspace=ws)
        torch.cuda.synchronize()
        _check(q, k, v, sl, 0, "bf16", out, tau)


def test_decode_rejects_small_workspace():
    # the binding refuses it before any launch (the C ABI's own rejection of
    # a small workspace is tested on the CPU)
    from entmax_amd import decode_workspace_bytes, entmax_attn_decode
    q, k, v, sl = _inputs(2, 4, 4, 64, 64, "f32", 1.0, seed=1, seqlens=[64, 10])
    ws = torch.empty((decode_workspace_bytes(2, 4, 4, 64, 64, 0, 1) - 256,), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        entmax_attn_decode(q.cuda(), k.cuda(), v.cuda(), sl.cuda(), 0, workspace=ws)


def test_decode_in_a_graph_replays_like_eager():
    # captured in a HIP graph (no memset nodes: the path writes every
    # workspace word it reads), every replay matches the eager call
    from entmax_amd import decode_workspace_bytes, entmax_attn_decode
    for S, window in ((2048, 32), (1100, 0)):
        q, k, v, sl = _inputs(4, 8, 2, S, 64, "bf16", 1.0, seed=S + window, seqlens=[S, 5, 0, S // 2])
        q, k, v, sl = q.cuda(), k.cuda(), v.cuda(), sl.cuda()
        log(f"[decode] graph S{S} W{window}")
        ws = torch.empty((decode_workspace_bytes(4, 8, 2, S, 64, window),), dtype=torch.uint8, device="cuda")
        ref_o, ref_t = entmax_attn_decode(q, k, v, sl, window, workspace=ws)
        out = torch.empty_like(ref_o)
        tau = torch.empty_like(ref_t)
        entmax_attn_decode(q, k, v, sl, window, out=out, tau=tau, workspace=ws)   # warm-up outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            entmax_attn_decode(q, k, v, sl, window, out=out, tau=tau, workspace=ws)
        for _ in range(3):
            out.fill_(7.0)
            tau.fill_(7.0)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o) and torch.equal(tau, ref_t)


MULTI = [
    # (dtype, d, H, Hkv, Lq, S, window)
    ("f32", 64, 4, 4, 2, 40, 32),
    ("bf16", 64, 8, 2, 5, 300, 32),
    ("bf16", 128, 8, 2, 5, 300, 0),
    ("f32", 64, 6, 3, 17, 600, 32),
    ("bf16", 64, 4, 1, 40, 700, 32),
    ("bf16", 64, 12, 12, 3, 2048, 0),
]


@pytest.mark.parametrize("dtype,d,H,Hkv,Lq,S,window", MULTI)
def test_decode_several_queries(dtype, d, H, Hkv, Lq, S, window):
    # Lq new tokens per sequence (query length below key length); the
    # shortest sequence holds fewer positions than queries
    from entmax_amd import entmax_attn_decode
    rng = np.random.default_rng(Lq * S + H)
    seqlens = [S, max(1, Lq // 2), int(rng.integers(Lq, S)), 0]
    gen = torch.Generator().manual_seed(S + Lq)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = torch.randn((4, H, Lq, d), generator=gen).to(dt)
    k = torch.randn((4, Hkv, S, d), generator=gen).to(dt)
    v = torch.randn((4, Hkv, S, d), generator=gen).to(dt)
    sl = torch.tensor(seqlens, dtype=torch.int32)
    log(f"[decode] {dtype} d{d} H{H} Hkv{Hkv} Lq{Lq} S{S} W{window} seqlens {seqlens}")
    out, tau = entmax_attn_decode(q.cuda(), k.cuda(), v.cuda(), sl.cuda(), window)
    torch.cuda.synchronize()
    assert out.shape == q.shape and tau.shape == q.shape[:-1]
    _check(q, k, v, sl, window, dtype, out, tau)


@pytest.mark.parametrize("name", ["decode", "decode_long"])
def test_decode_bench_workloads(name):
    # the inputs and launch configuration bench.py times, every row checked
    from entmax_amd import entmax_attn_decode
    from entmax_amd.workloads import make_decode_inputs
    inp = make_decode_inputs(name)
    w = inp["spec"]
    log(f"[decode] bench workload {name}")
    out, tau = entmax_attn_decode(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["seqlens"].cuda(),
                                  w["window"])
    torch.cuda.synchronize()
    _check(inp["q"], inp["k"], inp["v"], inp["seqlens"], w["window"], w["dtype"], out, tau)


@pytest.mark.parametrize("dtype,d,H,Hkv,Lq,S", [("f32", 64, 4, 2, 1, 200), ("bf16", 128, 8, 2, 5, 700),
                                              ("bf16", 64, 4, 4, 9, 3000)])
def test_decode_without_causal_mask(dtype, d, H, Hkv, Lq, S):
    # every cached key for every query (query length below key length, no mask)
    from entmax_amd import entmax_attn_decode
    seqlens = [S, 3, S // 2]
    gen = torch.Generator().manual_seed(S + 7 * Lq)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = torch.randn((3, H, Lq, d), generator=gen).to(dt)
    k = torch.randn((3, Hkv, S, d), generator=gen).to(dt)
    v = torch.randn((3, Hkv, S, d), generator=gen).to(dt)
    sl = torch.tensor(seqlens, dtype=torch.int32)
    log(f"[decode] no causal mask {dtype} d{d} H{H} Hkv{Hkv} Lq{Lq} S{S}")
    out, tau = entmax_attn_decode(q.cuda(), k.cuda(), v.cuda(), sl.cuda(), 0, causal=False)
    torch.cuda.synchronize()
    _check(q, k, v, sl, 0, dtype, out, tau, causal=False)


def test_decode_and_rows_are_deterministic():
    # no atomics and fixed summation orders: repeated calls give the same bits
    from entmax_amd import entmax15_rows, entmax_attn_decode
    q, k, v, sl = _inputs(2, 32, 8, 8192, 128, "bf16", 2.0, seed=11, seqlens=[8192, 4000])
    q, k, v, sl = q.cuda(), k.cuda(), v.cuda(), sl.cuda()
    o1, t1 = entmax_attn_decode(q, k, v, sl, 0)
    o2, t2 = entmax_attn_decode(q, k, v, sl, 0)
    s = torch.randn((40, 5000), generator=torch.Generator().manual_seed(3)).cuda()
    p1, u1 = entmax15_rows(s)
    p2, u2 = entmax15_rows(s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(t1, t2)
    assert torch.equal(p1, p2) and torch.equal(u1, u2)


# ---- backward at query length below key length (entmax_attn_decode_bwd) ----

DEC_BWD_CASES = [
    # B, H, Hkv, Lq, S, d, dtype, causal, window, seqlens
    (2, 4, 2, 1, 300, 64, "bf16", True, 0, [300, 177]),
    (2, 4, 2, 1, 300, 64, "bf16", True, 32, [300, 177]),
    (1, 2, 2, 5, 700, 128, "f32", True, 0, [650]),
    (2, 2, 1, 7, 520, 64, "f32", False, 0, [520, 301]),
    (1, 4, 1, 3, 3000, 128, "bf16", True, 0, [2990]),
    (1, 2, 2, 64, 64, 64, "f32", True, 0, [64]),
]


@pytest.mark.parametrize("case", DEC_BWD_CASES, ids=[f"c{i}" for i in range(len(DEC_BWD_CASES))])
def test_decode_backward(case):
    # dq, dk and dv after the kernel's own forward, against the float64
    # oracle's gradient; errors scaled by max(1, |reference|_inf)
    from entmax_amd import entmax_attn_decode, entmax_attn_decode_bwd
    from oracle import attention_decode_backward
    B, H, Hkv, Lq, S, d, dtype, causal, window, seqlens = case
    gen = torch.Generator().manual_seed(7000 + S + Lq)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = (torch.randn((B, H, Lq, d), generator=gen) * 1.5).to(dt)
    k = torch.randn((B, Hkv, S, d), generator=gen).to(dt)
    v = torch.randn((B, Hkv, S, d), generator=gen).to(dt)
    do = torch.randn((B, H, Lq, d), generator=gen).to(dt)
    sl = torch.tensor(seqlens, dtype=torch.int32)
    log(f"[decode bwd] B{B} H{H}/{Hkv} Lq{Lq} S{S} d{d} {dtype} causal {causal} window {window} seqlens {seqlens}")
    g = {n: x.cuda() for n, x in (("q", q), ("k", k), ("v", v), ("do", do), ("sl", sl))}
    _, tau = entmax_attn_decode(g["q"], g["k"], g["v"], g["sl"], window, causal=causal)
    dq, dk, dv = entmax_attn_decode_bwd(g["q"], g["k"], g["v"], g["sl"], tau, g["do"], window, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = attention_decode_backward(q, k, v, do, sl.numpy(), window, causal=causal)
    for name, x, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        err = float(np.abs(x.cpu().numpy() - r).max()) / max(1.0, float(np.abs(r).max()))
        log(f"[decode bwd]   scaled err {name} {err:.3g}")
        assert err <= TOL[dtype], (name, err)
    # deterministic: a second call gives the same bits
    dq2, dk2, dv2 = entmax_attn_decode_bwd(g["q"], g["k"], g["v"], g["sl"], tau, g["do"], window, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_decode_backward_rejects_small_workspace():
    from entmax_amd import decode_bwd_workspace_bytes, entmax_attn_decode, entmax_attn_decode_bwd
    q = torch.randn((1, 2, 1, 64), device="cuda")
    k = torch.randn((1, 2, 100, 64), device="cuda")
    sl = torch.tensor([100], dtype=torch.int32, device="cuda")
    _, tau = entmax_attn_decode(q, k, k, sl)
    need = decode_bwd_workspace_bytes(1, 2, 2, 100, 64, 0, 1)
    with pytest.raises(ValueError):
        entmax_attn_decode_bwd(q, k, k, sl, tau, q, workspace=torch.empty((need - 1,), dtype=torch.uint8, device="cuda"))
