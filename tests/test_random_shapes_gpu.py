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
    check_forward(inp, heads=head, check_probs=c["L"] <= 1024, label=label)
    if c["L"] <= 300:
        # grouped K, V: their gradients sum over every query head of the group
        check_backward(inp, heads=head if hkv == H else None, label=label)
