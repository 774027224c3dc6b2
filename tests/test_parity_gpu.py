"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bar (fixed by the method's target): absolute error <= 1e-5 for float32
inputs and <= 2e-3 for bfloat16 inputs on A, O and tau; the exact-zero
pattern of A must agree except for entries within 1e-6 of tau; backward
errors are scaled by max(1, |reference|_inf) with the same tolerance.
"""

import numpy as np
import pytest
import torch

from entmax_amd.workloads import WORKLOADS, make_inputs, random_inputs
from tests.parity_util import check_backward, check_forward, log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from entmax_amd import load_library
    load_library()


# ---- the named workloads ------------------------------------------------------

def test_tiny_full():
    check_forward(make_inputs("tiny"), label="tiny")


def test_encoder_full():
    check_forward(make_inputs("encoder"), label="encoder")


def test_long_subset_heads_full_rows():
    inp = make_inputs("long")
    # one head of every temperature (h = 0..11) for batch 0, all rows
    check_forward(inp, heads=[(0, h) for h in range(12)], label="long")


def test_long_sampled_rows_all_heads():
    inp = make_inputs("long")
    rows = np.array([0, 1, 511, 777, 1023])
    check_forward(inp, rows=rows, label="long/rows", check_probs=False)


def test_decoder_subset():
    inp = make_inputs("decoder")
    check_forward(inp, heads=[(0, 0), (3, 5), (7, 11)], label="decoder")


def test_decoder_sampled_rows_all_heads():
    inp = make_inputs("decoder")
    rows = np.array([0, 1, 31, 32, 33, 1000, 2047])
    check_forward(inp, rows=rows, label="decoder/rows", check_probs=False)


def test_longctx_forward_two_heads():
    # two whole heads: O, tau, A entry by entry and the exact-zero pattern
    inp = make_inputs("longctx")
    check_forward(inp, heads=[(0, 0), (0, 31)], label="longctx")


def test_longctx_forward_sampled_rows():
    inp = make_inputs("longctx")
    rows = np.array([0, 4095, 8191])
    check_forward(inp, heads=[(0, h) for h in range(0, 32, 3)], rows=rows, label="longctx/rows",
                  check_probs=False)


def test_longctx_backward_two_heads():
    inp = make_inputs("longctx")
    check_backward(inp, heads=[(0, 0), (0, 17)], label="longctx")


# ---- ragged shapes, masks, both dtypes and head dims ---------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L", [1, 7, 64, 100, 257])
def test_ragged_bidirectional(dtype, d, L):
    inp = random_inputs(2, 3, L, d, dtype, seed=L * 7 + d)
    check_forward(inp, label=f"ragged L{L}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gain", [0.05, 0.2, 0.3, 0.5])
@pytest.mark.parametrize("L", [300, 600])
def test_dense_supports_long(dtype, gain, L):
    # low-variance rows: hundreds of keys in the support, band lists near and
    # over capacity on the long-span path
    inp = random_inputs(1, 2, L, 64, dtype, seed=int(gain * 100) + L, qk_gain=gain)
    check_forward(inp, label=f"dense support gain{gain} L{L}")


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 1), (True, 5), (True, 32), (True, 100)])
@pytest.mark.parametrize("L", [50, 300, 1100])
def test_causal_and_window(causal, window, L):
    inp = random_inputs(1, 2, L, 64, "bf16", seed=L + window)
    inp["causal"], inp["window"] = causal, window
    check_forward(inp, label=f"causal w{window} L{L}", check_probs=L <= 300)


def test_padding_with_empty_sequences():
    inp = random_inputs(4, 2, 96, 64, "bf16", seed=5, key_lengths=[0, 1, 50, 96])
    errs, out, tau = check_forward(inp, label="padding")
    assert torch.all(out[0] == 0) and torch.all(torch.isinf(tau[0]))


def test_scattered_key_mask_causal():
    inp = random_inputs(2, 2, 200, 128, "f32", seed=6, key_mask_density=0.5)
    inp["causal"] = True
    check_forward(inp, label="scattered mask")


# ---- the streaming path (key span > 2048) and its overflow fallback -------------

def test_stream_path_bidirectional():
    inp = random_inputs(1, 2, 2200, 64, "bf16", seed=7)
    check_forward(inp, label="stream")


def test_stream_path_masked_f32():
    inp = random_inputs(2, 1, 2300, 128, "f32", seed=8, key_lengths=[2300, 2203])
    check_forward(inp, label="stream f32")


def test_stream_path_causal_window_and_grouped():
    # causal rows of up to 4000 keys with a wide window, grouped K and V
    inp = random_inputs(1, 4, 4000, 128, "bf16", seed=14, qk_gain=1.5)
    inp["k"], inp["v"] = inp["k"][:, :2].contiguous(), inp["v"][:, :2].contiguous()
    inp["causal"], inp["window"] = True, 2500
    check_forward(inp, heads=[(0, 0), (0, 3)], label="stream causal window gqa")

@pytest.mark.parametrize("dtype,d,causal", [("bf16", 64, False), ("f32", 128, True)])
def test_maximum_length(dtype, d, causal):
    # L = 65536, the largest length the entry points accept (the candidate
    # lists hold key indices as 16-bit integers): rows at both ends and in
    # the middle; the last causal row attends every key, 65535 included
    # float32 keeps scores of order one (the 1e-5 bar is its limit there);
    # its rows then overflow the candidate lists and take the fallback
    inp = random_inputs(1, 1, 65536, d, dtype, seed=65536 + d, qk_gain=1.5 if dtype == "bf16" else 1.0)
    inp["causal"] = causal
    rows = np.array([0, 1, 2047, 32768, 65534, 65535])
    check_forward(inp, rows=rows, label=f"max length {dtype} d{d}", check_probs=False)


def test_backward_maximum_length():
    # L = 65536 backward.  The full oracle gradient needs every (query, key)
    # pair; what any size allows instead:
    #  * dQ_i depends on row i alone: the oracle's row backward (alpha = 1.5)
    #    on the scores of sampled rows, dp_i = V dO_i, dQ_i = d^-1/2 dS_i K;
    #  * sum_j dK_j = 0 (every row of dS sums to zero: sum w (dp - c) = 0);
    #  * sum_j dV_j = sum_i dO_i (every row of p sums to one).
    from entmax_amd import entmax_attn_bwd, entmax_attn_fwd
    from oracle import entmax_alpha_backward
    from tests.parity_util import scores64, to_gpu
    L, d = 65536, 64
    inp = random_inputs(1, 1, L, d, "bf16", seed=77, qk_gain=1.5)
    g = to_gpu(inp)
    log("[parity] bwd max length bf16 d64 L65536")
    _, tau = entmax_attn_fwd(g["q"], g["k"], g["v"])
    dq, dk, dv = entmax_attn_bwd(g["q"], g["k"], g["v"], tau, g["dout"])
    torch.cuda.synchronize()
    k64 = inp["k"][0, 0].double().numpy()
    v64 = inp["v"][0, 0].double().numpy()
    do64 = inp["dout"][0, 0].double().numpy()
    rows = np.array([0, 1, 32768, 65535])
    s = scores64(inp["q"], inp["k"], 0, 0, rows)
    ds = entmax_alpha_backward(s, do64[rows] @ v64.T, 1.5)
    dq_ref = (ds @ k64) / np.sqrt(d)
    err = float(np.abs(dq.cpu().numpy()[0, 0][rows] - dq_ref).max()) / max(1.0, float(np.abs(dq_ref).max()))
    dk_c, dv_c = dk[0, 0].double().cpu().numpy(), dv[0, 0].double().cpu().numpy()
    # sums over 65536 keys of float32 atomics: relative to the sum of magnitudes
    sum_dk = float(np.abs(dk_c.sum(axis=0)).max()) / float(np.abs(dk_c).sum(axis=0).max())
    sum_dv = float(np.abs(dv_c.sum(axis=0) - do64.sum(axis=0)).max()) / float(np.abs(do64).sum(axis=0).max())
    log(f"[parity]   dq scaled err {err:.3g}; |sum dK| {sum_dk:.3g}, |sum dV - sum dO| {sum_dv:.3g} (relative)")
    assert err <= 2e-3
    assert sum_dk <= 1e-6 and sum_dv <= 1e-6


def test_stream_overflow_fallback():
    # near-uniform rows of 2200 keys: every key is a candidate, far more than
    # a list holds
    inp = random_inputs(1, 2, 2200, 64, "bf16", seed=9, qk_gain=0.2)
    check_forward(inp, label="stream overflow")


def _one_lane_flat_top(seed, d):
    """Rows of 2304 keys whose top is 576 near-equal scores, all on keys j
    with j % 16 < 4: the keys a single lane of a row holds in the wide
    forward, so that lane's list overflows while the row's other lanes hold
    few candidates."""
    inp = random_inputs(1, 1, 2304, d, "bf16", seed=seed)
    gen = torch.Generator().manual_seed(seed + 1)
    u = torch.randn(d, generator=gen)
    u = u * (8.0 / u.norm())
    q = (u + 0.3 * torch.randn(1, 1, 2304, d, generator=gen)).to(torch.bfloat16)
    k = inp["k"].float()
    sel = (torch.arange(2304) % 16) < 4
    k[:, :, sel] = u + 0.05 * torch.randn(1, 1, int(sel.sum()), d, generator=gen)
    return dict(inp, q=q, k=k.to(torch.bfloat16))


@pytest.mark.parametrize("d", [64, 128])
def test_wide_one_lane_overflow(d):
    from entmax_amd import entmax_attn_fwd_save
    from tests.parity_util import to_gpu
    inp = _one_lane_flat_top(41, d)
    g = to_gpu(inp)
    _, _, saved = entmax_attn_fwd_save(g["q"], g["k"], g["v"])
    torch.cuda.synchronize()
    counts = saved[: 2304 * 4].view(torch.int32).cpu()
    assert int((counts < 0).sum()) > 0, "no row took the overflow path"
    check_forward(inp, rows=np.arange(0, 2304, 37), label="one-lane overflow")
    check_backward(inp, label="one-lane overflow", saved=True)


def test_wide_lists_past_lds():
    # a flat top of 40 near-equal scores on keys spread over a row's lanes:
    # about ten candidates per lane, more than a lane keeps in LDS (the rest
    # go to the row's output row) and fewer than its list holds (no fix-up)
    from entmax_amd import entmax_attn_fwd_save
    from tests.parity_util import to_gpu
    inp = random_inputs(1, 1, 2304, 128, "bf16", seed=43)
    gen = torch.Generator().manual_seed(44)
    u = torch.randn(128, generator=gen)
    u = u * (8.0 / u.norm())
    q = (u + 0.3 * torch.randn(1, 1, 2304, 128, generator=gen)).to(torch.bfloat16)
    k = inp["k"].float()
    top = torch.randperm(2304, generator=gen)[:40]
    k[:, :, top] = u + 0.05 * torch.randn(1, 1, 40, 128, generator=gen)
    inp = dict(inp, q=q, k=k.to(torch.bfloat16))
    g = to_gpu(inp)
    _, _, saved = entmax_attn_fwd_save(g["q"], g["k"], g["v"])
    torch.cuda.synchronize()
    counts = saved[: 2304 * 4].view(torch.int32).cpu()
    assert int((counts < 0).sum()) == 0 and int(counts.max()) > 20, (int(counts.min()), int(counts.max()))
    check_forward(inp, rows=np.arange(0, 2304, 37), label="lists past LDS")
    check_backward(inp, label="lists past LDS", saved=True)


# ---- determinism and streams ----------------------------------------------------

def test_forward_is_deterministic():
    from entmax_amd import entmax_attn_fwd
    inp = make_inputs("encoder")
    q, k, v, km = (inp[x].cuda() for x in ("q", "k", "v", "key_mask"))
    o1, t1 = entmax_attn_fwd(q, k, v, km)
    o2, t2 = entmax_attn_fwd(q, k, v, km)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(t1, t2)


@pytest.mark.parametrize("gain", [2.0, 0.4])
def test_wide_forward_is_deterministic(gain):
    # spans beyond 2048 keys: each lane of a row keeps its own candidates,
    # in a fixed order; gain 0.4 also overflows lists (the fix-up)
    from entmax_amd import entmax_attn_fwd
    from tests.parity_util import to_gpu
    g = to_gpu(random_inputs(1, 2, 2304, 128, "bf16", seed=21, qk_gain=gain))
    o1, t1 = entmax_attn_fwd(g["q"], g["k"], g["v"])
    o2, t2 = entmax_attn_fwd(g["q"], g["k"], g["v"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(t1, t2)


def test_runs_on_a_side_stream():
    from entmax_amd import entmax_attn_fwd
    inp = random_inputs(2, 2, 256, 64, "bf16", seed=10)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    ref, _ = entmax_attn_fwd(q, k, v)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, _ = entmax_attn_fwd(q, k, v)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


# ---- backward on small cases ------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_small(dtype):
    inp = random_inputs(2, 2, 77, 64, dtype, seed=11, qk_gain=1.5)
    check_backward(inp, label="small")


def test_backward_masked_causal_window():
    inp = random_inputs(2, 2, 150, 128, "bf16", seed=12, key_lengths=[150, 90])
    inp["causal"], inp["window"] = True, 32
    check_backward(inp, label="masked causal window")


def test_backward_dense_support_overflow():
    # supports of hundreds of keys: the per-row list overflows; the key side
    # flushes its lists many times per key
    inp = random_inputs(1, 2, 600, 64, "f32", seed=13, qk_gain=0.3)
    check_backward(inp, label="dense support")


@pytest.mark.parametrize("L,gain,causal", [(2304, 2.0, False), (2400, 0.4, False), (3000, 1.0, True)])
def test_backward_long_spans(L, gain, causal):
    # spans beyond 2048 keys take the wide query-side kernel; gain 0.4 gives
    # supports of hundreds of keys (overflow markers and the tile fix-up)
    inp = random_inputs(1, 2, L, 128, "bf16", seed=L + 3, qk_gain=gain)
    inp["causal"] = causal
    check_backward(inp, label=f"long span gain{gain}")


def test_backward_long_span_f32_masked_window():
    inp = random_inputs(2, 1, 2600, 64, "f32", seed=15, key_lengths=[2600, 2311])
    inp["causal"], inp["window"] = True, 2200
    check_backward(inp, label="long span f32 masked window")


# ---- backward on the support the forward kept ------------------------------------

@pytest.mark.parametrize("L,d,dtype,gain,causal,window,lengths", [
    (2304, 128, "bf16", 2.0, False, 0, None),       # wide: every row kept
    (2400, 128, "bf16", 0.4, False, 0, None),       # supports of hundreds: rows not kept, fix-up
    (3000, 128, "bf16", 1.0, True, 0, None),        # causal, ragged tail of rows
    (2600, 64, "f32", 1.0, True, 2200, [2600, 2311]),   # window, key padding, float32
    (300, 64, "bf16", 1.5, False, 0, None),         # short span: the buffer is not used
])
def test_backward_on_saved_support(L, d, dtype, gain, causal, window, lengths):
    B = 1 if lengths is None else len(lengths)
    inp = random_inputs(B, 2, L, d, dtype, seed=L + 31, qk_gain=gain, key_lengths=lengths)
    inp["causal"], inp["window"] = causal, window
    check_backward(inp, label=f"saved support gain{gain}", saved=True)


def test_backward_on_saved_support_grouped_and_repeatable():
    from entmax_amd import entmax_attn_bwd_saved, entmax_attn_fwd_save
    from tests.parity_util import to_gpu
    inp = random_inputs(1, 4, 2304, 64, "bf16", seed=41, qk_gain=2.0)
    inp["k"], inp["v"] = inp["k"][:, :2].contiguous(), inp["v"][:, :2].contiguous()   # two key/value heads
    check_backward(inp, label="saved support grouped", saved=True)
    g = to_gpu(inp)
    _, tau, sv = entmax_attn_fwd_save(g["q"], g["k"], g["v"])
    a = entmax_attn_bwd_saved(g["q"], g["k"], g["v"], tau, g["dout"], sv)
    b = entmax_attn_bwd_saved(g["q"], g["k"], g["v"], tau, g["dout"], sv)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("L,d,gain", [(300, 64, 1.5), (2304, 128, 2.0), (2200, 64, 0.3)])
def test_backward_is_deterministic(L, d, gain):
    # query rows and key rows each have one owner and a fixed summation
    # order: two calls give identical bits
    from entmax_amd import entmax_attn_bwd, entmax_attn_fwd
    from tests.parity_util import to_gpu
    g = to_gpu(random_inputs(2, 2, L, d, "bf16", seed=L + d, qk_gain=gain))
    _, tau = entmax_attn_fwd(g["q"], g["k"], g["v"])
    a = entmax_attn_bwd(g["q"], g["k"], g["v"], tau, g["dout"])
    b = entmax_attn_bwd(g["q"], g["k"], g["v"], tau, g["dout"])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_plain_entry_points_through_ctypes():
    # entmax_attn_fwd / entmax_attn_bwd (not the grouped variants) called
    # with raw pointers, against the oracle
    import ctypes
    from entmax_amd import bwd_workspace_bytes, load_library
    from oracle import attention_backward, attention_forward
    from tests.parity_util import to_gpu
    lib = load_library()
    inp = random_inputs(2, 2, 150, 64, "bf16", seed=21, key_lengths=[150, 97])
    g = to_gpu(inp)
    B, H, L, d = g["q"].shape
    out = torch.empty((B, H, L, d), device="cuda")
    tau = torch.empty((B, H, L), device="cuda")
    grads = [torch.empty((B, H, L, d), device="cuda") for _ in range(3)]
    ws = torch.empty((bwd_workspace_bytes(B, H, L, d),), dtype=torch.uint8, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.entmax_attn_fwd(P(g["q"]), P(g["k"]), P(g["v"]), P(g["key_mask"]), 0, 0, P(out), P(tau),
                               B, H, L, d, 1, st) == 0
    assert lib.entmax_attn_bwd(P(g["q"]), P(g["k"]), P(g["v"]), P(g["key_mask"]), 0, 0, P(tau), P(g["dout"]),
                               P(grads[0]), P(grads[1]), P(grads[2]), B, H, L, d, 1, P(ws), ws.numel(), st) == 0
    torch.cuda.synchronize()
    ref = attention_forward(inp["q"], inp["k"], inp["v"], inp["key_mask"])
    refb = attention_backward(inp["q"], inp["k"], inp["v"], inp["dout"], inp["key_mask"])
    assert float(np.abs(out.cpu().numpy().reshape(ref["out"].shape) - ref["out"]).max()) <= 2e-3
    for name, gt in zip(("dq", "dk", "dv"), grads):
        r = refb[name]
        err = float(np.abs(gt.cpu().numpy().reshape(r.shape) - r).max()) / max(1.0, float(np.abs(r).max()))
        assert err <= 2e-3, (name, err)


# ---- grouped-query attention (key/value heads shared by groups of query heads) ----

def _grouped(inp, hkv):
    out = dict(inp)
    out["k"] = inp["k"][:, :hkv].contiguous()
    out["v"] = inp["v"][:, :hkv].contiguous()
    return out


@pytest.mark.parametrize("L,dtype,hkv", [(128, "bf16", 1), (100, "f32", 2), (600, "bf16", 2), (2200, "bf16", 1)])
def test_grouped_query_forward(L, dtype, hkv):
    # spans of <= 128, 129..2048 and > 2048 keys: the three forward kernels
    inp = _grouped(random_inputs(2, 4, L, 64, dtype, seed=31, qk_gain=1.2, key_lengths=[L, L - L // 3]), hkv)
    heads = None if L <= 600 else [(0, 0), (0, 3), (1, 1)]
    check_forward(inp, heads=heads, label=f"gqa H4/Hkv{hkv}", check_probs=L <= 600)


def test_grouped_query_causal_window_forward():
    inp = _grouped(random_inputs(2, 6, 300, 128, "bf16", seed=32), 3)
    inp["causal"], inp["window"] = True, 32
    check_forward(inp, label="gqa causal window")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grouped_query_backward(dtype):
    # dk, dv of a shared head collect the atomics of all its query heads
    inp = _grouped(random_inputs(2, 4, 90, 64, dtype, seed=33, qk_gain=1.5, key_lengths=[90, 61]), 2)
    check_backward(inp, label="gqa")


@pytest.mark.parametrize("L,causal", [(128, False), (128, True), (199, True), (600, False)])
def test_dense_rows_with_one_high_key(L, causal):
    # nearly every key in the support and one key well above the rest: after
    # the first bisection stage a lane can still hold more than 16 band
    # entries, which the exact finish must not truncate
    inp = random_inputs(1, 2, L, 64, "f32", seed=L + int(causal), qk_gain=0.3)
    qm = inp["q"][0, 0].mean(0)
    inp["k"][0, :, L // 2] += 4.0 * qm / (qm.norm() ** 2)
    inp["causal"] = causal
    check_forward(inp, label=f"dense + one high key L{L} causal={causal}")


def test_binding_refuses_bad_outputs_before_launch():
    # outputs, tau and workspaces of the wrong shape, dtype, device or layout
    # raise ValueError in the binding; nothing reaches the kernels
    from entmax_amd import entmax_attn_bwd, entmax_attn_fwd, entmax_attn_probs
    from tests.parity_util import to_gpu
    g = to_gpu(random_inputs(1, 2, 64, 64, "bf16", seed=3))
    q, k, v, do = g["q"], g["k"], g["v"], g["dout"]
    out, tau = entmax_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    bad_out = [torch.empty((1, 2, 64, 32), device="cuda"), torch.empty((1, 2, 64, 64), device="cuda",
                                                                       dtype=torch.bfloat16),
               torch.empty((1, 2, 64, 64)), torch.empty((1, 2, 64, 64), device="cuda").transpose(2, 3)]
    for o in bad_out:
        with pytest.raises(ValueError):
            entmax_attn_fwd(q, k, v, out=o)
    with pytest.raises(ValueError):
        entmax_attn_fwd(q, k, v, tau_out=torch.empty((1, 2, 63), device="cuda"))
    with pytest.raises(ValueError):
        entmax_attn_bwd(q, k, v, tau.cpu(), do)                                  # tau on the CPU
    with pytest.raises(ValueError):
        entmax_attn_bwd(q, k, v, tau, do, dk=torch.empty((1, 2, 64, 64), device="cuda", dtype=torch.float16))
    with pytest.raises(ValueError):
        entmax_attn_bwd(q, k, v, tau, do, workspace=torch.empty((4,), dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        entmax_attn_probs(q, k, tau, probs=torch.empty((1, 2, 64, 32), device="cuda"))
    torch.cuda.synchronize()
