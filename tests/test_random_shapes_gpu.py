"""GPU parity on seeded random shapes: batch, heads, length (short, long and
stream paths), head dimension, dtype, causal mask and window, padding and
score scale drawn from a fixed generator, forward checked on every row of
one head per case, backward on the short cases.  Same bar as
test_parity_gpu.py."""

import numpy as np
import pytest
import torch

from entmax_amd.workloads import random_inputs
from tests.parity_util import check_backward, check_forward

pytestmark = pytest.mark.gpu


def _cases(n=20, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        band = i % 3
        L = int(rng.integers(1, 129) if band == 0 else rng.integers(129, 1025) if band == 1 else rng.integers(1025, 2500))
        causal = bool(rng.random() < 0.5)
        window = int(rng.choice([0, 1, 7, 32, 100])) if causal else 0
        out.append(dict(B=int(rng.integers(1, 4)), H=int(rng.integers(1, 4)), L=L, d=int(rng.choice([64, 128])),
                        dtype=str(rng.choice(["f32", "bf16"])), causal=causal, window=window,
                        pad=str(rng.choice(["none", "right", "scattered"])), gain=float(rng.choice([0.3, 1.0, 2.0])),
                        seed=1000 + i))
    return out


CASES = _cases()


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
    inp = random_inputs(c["B"], c["H"], c["L"], c["d"], c["dtype"], seed=c["seed"], qk_gain=c["gain"], **kw)
    inp["causal"], inp["window"] = c["causal"], c["window"]
    label = (f"random B{c['B']} H{c['H']} L{c['L']} d{c['d']} {c['dtype']} causal={c['causal']} "
             f"W{c['window']} pad={c['pad']} gain={c['gain']}")
    head = [(c["B"] - 1, c["H"] - 1)]
    check_forward(inp, heads=head, check_probs=c["L"] <= 1024, label=label)
    if c["L"] <= 300:
        check_backward(inp, heads=head, label=label)
