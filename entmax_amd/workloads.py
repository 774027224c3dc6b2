"""Seeded synthetic inputs for 1.5-entmax attention.

This module only draws random tensors; it holds none of the method's
arithmetic.  Both the HIP path (tests, bench) and the float64 oracle take
their inputs from here, so the two sides see the same bytes.

Recipe (one generator per workload, CPU, ``torch.Generator`` seeded with
1000 + workload number): draw float32 ``randn`` for Q, K, V and dO in that
order, then the per-sequence lengths or per-head temperatures, apply the
workload's scaling, then cast to the workload's dtype.  The cast tensors are
what both sides consume (the oracle upcasts them exactly).

Workloads (shapes, distributions and masks of the pages' encoder and decoder
settings; no dataset is used):

* ``tiny``      B2 H2 L64 d64 fp32, N(0,1), no mask.
* ``encoder``   B32 H12 L128 d64 bf16, N(0,1), right padding: sequence b has
  a valid length drawn uniformly from [8, 128]; keys past it are masked.
  Stands in for the RoBERTa-base SST-2 batches (L=128, B=32, 12 heads, d=64).
* ``long``      B8 H12 L1024 d64 bf16; head h draws a temperature T_h uniform
  in [1, 3] (shared over the batch) and both Q and K are divided by it.
* ``decoder``   B8 H12 L2048 d64 bf16, N(0,1), causal with a 32-key window.
* ``longctx``   B1 H32 L8192 d128 bf16, Q and K times 2, V and dO N(0,1);
  forward and backward.

Decode time (``make_decode_inputs``): one new query per sequence against a
full key/value cache, q [B, H, d], caches [B, H, S, d], seqlens = S:

* ``decode``       the decoder workload's shape (B8 H12 S2048 d64 bf16,
  N(0,1)) with its 32-key window; seed 1007.
* ``decode_long``  the long-context shape (B1 H32 S8192 d128 bf16, q and k
  times 2) without a window, every cached key allowed; seed 1008.

Row-wise op (``make_row_inputs``): ``rows`` is a [98304, 1024] bf16 score
matrix (the rows of the long workload's 8 x 12 heads) drawn N(0,1), with a
float32 N(0,1) gradient for the backward; seed 1006.
"""

from dataclasses import dataclass, field
from typing import Optional

import torch

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    number: int
    B: int
    H: int
    L: int
    d: int
    dtype: str
    causal: bool = False
    window: int = 0
    padding: bool = False          # right padding with lengths U[8, L]
    temperature: Optional[tuple] = None   # (lo, hi): Q, K divided by T_h
    qk_gain: float = 1.0           # Q and K multiplied by this
    backward: bool = False
    notes: str = ""


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, 2, 2, 64, 64, "f32"),
        Workload("encoder", 2, 32, 12, 128, 64, "bf16", padding=True),
        Workload("long", 3, 8, 12, 1024, 64, "bf16", temperature=(1.0, 3.0)),
        Workload("decoder", 4, 8, 12, 2048, 64, "bf16", causal=True, window=32),
        Workload("longctx", 5, 1, 32, 8192, 128, "bf16", qk_gain=2.0, backward=True),
    ]
}


def make_inputs(name, device="cpu", seed=None):
    """Draw the inputs of a named workload.

    Returns a dict: q, k, v, dout ([B, H, L, d], workload dtype), key_mask
    ([B, L] uint8, or None), causal, window, plus 'lengths' / 'temperature'
    when drawn.  Tensors are created on the CPU and then moved to ``device``.
    """
    w = WORKLOADS[name]
    gen = torch.Generator().manual_seed(1000 + w.number if seed is None else seed)
    shape = (w.B, w.H, w.L, w.d)
    q = torch.randn(shape, generator=gen)
    k = torch.randn(shape, generator=gen)
    v = torch.randn(shape, generator=gen)
    dout = torch.randn(shape, generator=gen)
    out = {"causal": w.causal, "window": w.window, "key_mask": None, "workload": w}
    if w.padding:
        lengths = torch.randint(8, w.L + 1, (w.B,), generator=gen)
        out["lengths"] = lengths
        out["key_mask"] = (torch.arange(w.L)[None, :] < lengths[:, None]).to(torch.uint8)
    if w.temperature is not None:
        lo, hi = w.temperature
        t = lo + (hi - lo) * torch.rand(w.H, generator=gen)
        out["temperature"] = t
        q = q / t[None, :, None, None]
        k = k / t[None, :, None, None]
    if w.qk_gain != 1.0:
        q = q * w.qk_gain
        k = k * w.qk_gain
    dt = _DTYPES[w.dtype]
    for name_, x in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        out[name_] = x.to(dt).contiguous().to(device)
    if out["key_mask"] is not None:
        out["key_mask"] = out["key_mask"].to(device)
    return out


def random_inputs(B, H, L, d, dtype="bf16", seed=0, qk_gain=1.0, key_lengths=None,
                  key_mask_density=None, device="cpu"):
    """Generic seeded inputs for parity cases of arbitrary shape.

    ``key_lengths``: per-sequence valid lengths (right padding); or
    ``key_mask_density``: each key kept independently with that probability
    (scattered padding).  Returns the same dict layout as ``make_inputs``.
    """
    gen = torch.Generator().manual_seed(seed)
    shape = (B, H, L, d)
    q = torch.randn(shape, generator=gen) * qk_gain
    k = torch.randn(shape, generator=gen) * qk_gain
    v = torch.randn(shape, generator=gen)
    dout = torch.randn(shape, generator=gen)
    km = None
    if key_lengths is not None:
        lengths = torch.as_tensor(key_lengths)
        km = (torch.arange(L)[None, :] < lengths[:, None]).to(torch.uint8)
    elif key_mask_density is not None:
        km = (torch.rand((B, L), generator=gen) < key_mask_density).to(torch.uint8)
    dt = _DTYPES[dtype]
    res = {"key_mask": None if km is None else km.to(device), "causal": False, "window": 0}
    for name_, x in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        res[name_] = x.to(dt).contiguous().to(device)
    return res


ROWS = {"rows": {"R": 98304, "L": 1024, "dtype": "bf16", "number": 6}}


def make_row_inputs(name="rows", device="cpu"):
    """Scores [R, L] (workload dtype) and an incoming gradient [R, L] float32."""
    w = ROWS[name]
    gen = torch.Generator().manual_seed(1000 + w["number"])
    s = torch.randn((w["R"], w["L"]), generator=gen)
    dp = torch.randn((w["R"], w["L"]), generator=gen)
    return {"scores": s.to(_DTYPES[w["dtype"]]).contiguous().to(device), "dp": dp.to(device), "spec": w}



DECODE = {
    "decode": {"B": 8, "H": 12, "Hkv": 12, "S": 2048, "d": 64, "dtype": "bf16", "window": 32,
               "qk_gain": 1.0, "number": 7},
    "decode_long": {"B": 1, "H": 32, "Hkv": 32, "S": 8192, "d": 128, "dtype": "bf16", "window": 0,
                    "qk_gain": 2.0, "number": 8},
}


def make_decode_inputs(name, device="cpu"):
    """q [B, H, d], k_cache, v_cache [B, H_kv, S, d] (workload dtype) and
    seqlens [B] int32 (every cache full)."""
    w = DECODE[name]
    gen = torch.Generator().manual_seed(1000 + w["number"])
    q = torch.randn((w["B"], w["H"], w["d"]), generator=gen) * w["qk_gain"]
    k = torch.randn((w["B"], w["Hkv"], w["S"], w["d"]), generator=gen) * w["qk_gain"]
    v = torch.randn((w["B"], w["Hkv"], w["S"], w["d"]), generator=gen)
    dt = _DTYPES[w["dtype"]]
    seqlens = torch.full((w["B"],), w["S"], dtype=torch.int32)
    return {"q": q.to(dt).to(device), "k": k.to(dt).to(device), "v": v.to(dt).to(device),
            "seqlens": seqlens.to(device), "spec": w}
