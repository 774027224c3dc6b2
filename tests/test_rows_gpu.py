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
@pytest.mark.parametrize("L,gain", [(4, 1.0), (100, 2.0), (256, 0.5), (1000, 4.0), (4096, 1.0), (4100, 3.0), (6000, 0.3)])
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
