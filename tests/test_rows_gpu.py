"""GPU parity of the row-wise 1.5-entmax op (entmax15_rows_fwd / _bwd through
the C ABI) against the float64 oracle: absolute error <= 1e-5 (float32
scores) or 2e-3 (bfloat16 scores) on p and tau, the exact-zero pattern equal
except within 1e-6 of tau; the backward to the same tolerance, scaled by
max(1, |reference|_inf)."""

import numpy as np
import pytest
import torch

from oracle import entmax15_backward, entmax15_exact
from tests.parity_util import NEAR_TAU, TOL, log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _scores(R, L, dtype, gain, seed):
    gen = torch.Generator().manual_seed(seed)
    s = (torch.randn((R, L), generator=gen) * gain).to(torch.float32 if dtype == "f32" else torch.bfloat16)
    mask = (torch.rand((R, L), generator=gen) > 0.2).to(torch.uint8)
    mask[0] = 0            # a row with no allowed entry
    mask[1] = 1            # a row with all entries allowed
    return s, mask


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
# L = 40000 with fewer than 1024 rows: a workgroup per row, streamed from
# memory at every step (rows beyond the 16384 entries its registers hold)
@pytest.mark.parametrize("L,gain", [(4, 1.0), (100, 2.0), (256, 0.5), (1000, 4.0), (4096, 1.0), (4100, 3.0), (6000, 0.3),
                                    (40000, 1.0)])
def test_rows_forward(dtype, L, gain):
    from entmax_amd import entmax15_rows
    R = 37
    s, mask = _scores(R, L, dtype, gain, seed=L + int(10 * gain))
    log(f"[rows] fwd {dtype} R{R} L{L} gain {gain}")
    p, tau = entmax15_rows(s.cuda(), mask.cuda())
    torch.cuda.synchronize()
    s64 = s.to(torch.float64).numpy()
    ok = mask.numpy() != 0
    p_ref, tau_ref = entmax15_exact(s64, ok)
    p_c, tau_c = p.cpu().numpy(), tau.cpu().numpy()
    assert np.array_equal(np.isinf(tau_c), np.isinf(tau_ref))
    fin = np.isfinite(tau_ref)
    tol = TOL[dtype]
    err_p = float(np.abs(p_c - p_ref).max())
    err_t = float(np.abs(tau_c[fin] - tau_ref[fin]).max())
    near = np.abs(s64 - np.where(fin, tau_ref, 0.0)[:, None]) <= NEAR_TAU
    bad = int((((p_c == 0) != (p_ref == 0)) & ok & ~near).sum())
    log(f"[rows]   max err p={err_p:.3g} tau={err_t:.3g} pattern_bad={bad}")
    assert err_p <= tol and err_t <= tol and bad == 0
    assert np.all(p_c[~ok] == 0)
    np.testing.assert_allclose(p_c[fin].sum(axis=1), 1.0, atol=1e-4)


@pytest.mark.parametrize("L", [64, 1000, 5000])
def test_rows_backward(L):
    from entmax_amd import entmax15_rows, entmax15_rows_bwd
    R = 21
    s, mask = _scores(R, L, "f32", 2.0, seed=7 * L)
    dp = torch.randn((R, L), generator=torch.Generator().manual_seed(L))
    p, _ = entmax15_rows(s.cuda(), mask.cuda())
    ds = entmax15_rows_bwd(p, dp.cuda())
    torch.cuda.synchronize()
    ref = entmax15_backward(s.to(torch.float64).numpy(), dp.to(torch.float64).numpy(), mask.numpy() != 0)
    err = float(np.abs(ds.cpu().numpy() - ref).max()) / max(1.0, float(np.abs(ref).max()))
    log(f"[rows] bwd L{L} scaled err {err:.3g}")
    assert err <= TOL["f32"]


def test_rows_rejects_bad_shapes():
    from entmax_amd import EntmaxError, entmax15_rows
    with pytest.raises(EntmaxError):
        entmax15_rows(torch.zeros((3, 10), device="cuda"))   # L not a multiple of 4


# General alpha (entmax_bisect_rows_fwd / _bwd) against the float64 solve of
# entmax_alpha_exact.  The same tolerances hold: the kernel's error on p is
# about (1/(alpha-1)) times the float32 rounding of the scaled scores plus
# 2^-25 of the bracket, 1e-6 or less for alpha >= 1.1.  Exact p values below
# float32's normal range (tiny powers for alpha near 1) may flush to zero, so
# the zero pattern is compared where the exact p is zero or above 1e-30.
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("alpha", [1.1, 1.25, 1.75, 2.0])
@pytest.mark.parametrize("L,gain", [(100, 2.0), (1000, 1.0), (4100, 3.0), (40000, 1.0)])
def test_bisect_rows_forward(dtype, alpha, L, gain):
    from entmax_amd import entmax_bisect_rows
    from oracle import entmax_alpha_exact
    R = 19
    s, mask = _scores(R, L, dtype, gain, seed=3 * L + int(100 * alpha))
    log(f"[rows] alpha {alpha} fwd {dtype} R{R} L{L} gain {gain}")
    p, tau = entmax_bisect_rows(s.cuda(), alpha, mask.cuda())
    torch.cuda.synchronize()
    s64 = s.to(torch.float64).numpy()
    ok = mask.numpy() != 0
    p_ref, tau_ref = entmax_alpha_exact(s64, alpha, ok)
    p_c, tau_c = p.cpu().numpy(), tau.cpu().numpy()
    assert np.array_equal(np.isinf(tau_c), np.isinf(tau_ref))
    fin = np.isfinite(tau_ref)
    tol = TOL[dtype]
    err_p = float(np.abs(p_c - p_ref).max())
    err_t = float(np.abs(tau_c[fin] - tau_ref[fin]).max())
    near = np.abs(s64 - np.where(fin, tau_ref, 0.0)[:, None]) <= NEAR_TAU
    judged = ok & ~near & ((p_ref == 0) | (p_ref > 1e-30))
    bad = int((((p_c == 0) != (p_ref == 0)) & judged).sum())
    log(f"[rows]   max err p={err_p:.3g} tau={err_t:.3g} pattern_bad={bad}")
    assert err_p <= tol and err_t <= tol and bad == 0
    assert np.all(p_c[~ok] == 0)
    np.testing.assert_allclose(p_c[fin].sum(axis=1), 1.0, atol=1e-4)


def test_bisect_rows_alpha15_is_entmax15():
    # alpha = 1.5 through the general entry point runs the 1.5 kernels
    from entmax_amd import entmax15_rows, entmax_bisect_rows
    s, mask = _scores(8, 1000, "f32", 2.0, seed=1)
    p1, t1 = entmax15_rows(s.cuda(), mask.cuda())
    p2, t2 = entmax_bisect_rows(s.cuda(), 1.5, mask.cuda())
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(t1, t2)


@pytest.mark.parametrize("alpha", [1.25, 1.75, 2.0])
@pytest.mark.parametrize("L", [64, 5000])
def test_bisect_rows_backward(alpha, L):
    from entmax_amd import entmax_bisect_rows, entmax_bisect_rows_bwd
    from oracle import entmax_alpha_backward, entmax_alpha_exact
    R = 13
    s, mask = _scores(R, L, "f32", 2.0, seed=5 * L + int(10 * alpha))
    dp = torch.randn((R, L), generator=torch.Generator().manual_seed(L + 1))
    log(f"[rows] alpha {alpha} bwd L{L}")
    s64, ok = s.to(torch.float64).numpy(), mask.numpy() != 0
    ref = entmax_alpha_backward(s64, dp.to(torch.float64).numpy(), alpha, ok)
    # on the oracle's p (float32): the backward entry point's own parity
    p_ref, _ = entmax_alpha_exact(s64, alpha, ok)
    ds = entmax_bisect_rows_bwd(torch.from_numpy(p_ref).float().cuda(), dp.cuda(), alpha)
    torch.cuda.synchronize()
    err = float(np.abs(ds.cpu().numpy() - ref).max()) / max(1.0, float(np.abs(ref).max()))
    log(f"[rows]   scaled err on the oracle's p {err:.3g}")
    assert err <= TOL["f32"]
    # the chain after the kernel's own forward: against the exact backward at
    # the kernel's output p for every row, and against the exact backward for the
    # rows that are well conditioned at the measured tau error (all rows for
    # alpha <= 1.5; chain_rows_ok above)
    from oracle import entmax_alpha_vjp
    from tests.parity_util import chain_rows_ok
    p, tau = entmax_bisect_rows(s.cuda(), alpha, mask.cuda())
    ds = entmax_bisect_rows_bwd(p, dp.cuda(), alpha)
    torch.cuda.synchronize()
    dsn = ds.cpu().numpy()
    tg = tau.cpu().numpy().astype(np.float64)
    ref_at = entmax_alpha_vjp(p.cpu().numpy(), dp.to(torch.float64).numpy(), alpha)
    err = float(np.abs(dsn - ref_at).max()) / max(1.0, float(np.abs(ref_at).max()))
    log(f"[rows]   scaled err after the kernel's forward, at its p {err:.3g}")
    assert err <= TOL["f32"]
    _, t_ref = entmax_alpha_exact(s64, alpha, ok)
    keep, band = chain_rows_ok(s64, tg, t_ref, alpha, ok)
    if keep.any():
        err = float(np.abs(dsn[keep] - ref[keep]).max()) / max(1.0, float(np.abs(ref[keep]).max()))
        log(f"[rows]   scaled err after the kernel's forward {err:.3g} ({int(keep.sum())} of {R} rows)")
        assert err <= TOL["f32"]


def test_rows_bench_workload_sampled():
    # the [98304, 1024] score matrix bench.py times, 96 sampled rows checked
    from entmax_amd import entmax15_rows, entmax15_rows_bwd
    from entmax_amd.workloads import make_row_inputs
    inp = make_row_inputs("rows")
    log("[rows] bench workload R98304 L1024")
    s = inp["scores"].cuda()
    p, tau = entmax15_rows(s)
    ds = entmax15_rows_bwd(p, inp["dp"].cuda())
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(s.shape[0], 96, replace=False)
    s64 = inp["scores"][rows].to(torch.float64).numpy()
    p_ref, tau_ref = entmax15_exact(s64)
    assert float(np.abs(p.cpu().numpy()[rows] - p_ref).max()) <= TOL["bf16"]
    assert float(np.abs(tau.cpu().numpy()[rows] - tau_ref).max()) <= TOL["bf16"]
    ref = entmax15_backward(s64, inp["dp"][rows].to(torch.float64).numpy())
    err = float(np.abs(ds.cpu().numpy()[rows] - ref).max()) / max(1.0, float(np.abs(ref).max()))
    assert err <= TOL["f32"]
