"""The allocation-free backward (entmax_attn_bwd_noalloc) against the
backward with a caller workspace (entmax_attn_bwd_gqa), through the C ABI.

Both run the same deterministic kernels, so the gradients must agree bit for
bit.  The scratch is shared and keeps the last call's contents, so the check
runs two calls in a row, the second with a smaller input.
"""

import ctypes

import pytest
import torch

from entmax_amd.workloads import make_inputs, random_inputs

P8 = ctypes.c_void_p(256)   # an aligned stand-in pointer: never dereferenced by a rejected call


@pytest.fixture(scope="module")
def lib():
    from entmax_amd import load_library
    return load_library()


def test_noalloc_rejects_oversize_and_null(lib):
    # host-side checks only: these calls return before any GPU work
    # q, k, v, mask, causal, window, tau, dout, dq, dk, dv, B, H, H_kv, L, d, dtype, stream
    ok = [P8, P8, P8, None, 0, 0, P8, P8, P8, P8, P8, 1, 2, 2, 8, 64, 1, None]
    a = list(ok)
    a[11:15] = [4, 32, 32, 8193]                                  # 1048704 query rows > 1048576
    assert lib.entmax_attn_bwd_noalloc(*a) == 1
    assert b"scratch" in lib.entmax_attn_last_error()
    for i in (0, 1, 2, 6, 7, 8, 9, 10):                           # a required pointer missing
        a = list(ok)
        a[i] = None
        assert lib.entmax_attn_bwd_noalloc(*a) == 1, i
    a = list(ok)
    a[12:14] = [3, 2]                                             # H_kv does not divide H
    assert lib.entmax_attn_bwd_noalloc(*a) == 1
    a = list(ok)
    a[15] = 96                                                    # unsupported head dimension
    assert lib.entmax_attn_bwd_noalloc(*a) == 2


def _to_gpu(inp):
    out = {}
    for name in ("q", "k", "v", "dout"):
        out[name] = inp[name].to("cuda").contiguous()
    km = inp.get("key_mask")
    out["key_mask"] = None if km is None else km.to("cuda").contiguous()
    return out


def _both(lib, inp, causal=False, window=0):
    from entmax_amd import bwd_workspace_bytes, entmax_attn_fwd
    g = _to_gpu(inp)
    q, k, v, dout, km = g["q"], g["k"], g["v"], g["dout"], g["key_mask"]
    B, H, L, d = q.shape
    hkv = k.shape[1]
    _, tau = entmax_attn_fwd(q, k, v, key_mask=km, causal=causal, window=window)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    dt = 1 if q.dtype == torch.bfloat16 else 0
    ref = [torch.empty((B, h, L, d), device="cuda") for h in (H, hkv, hkv)]
    ws = torch.empty((bwd_workspace_bytes(B, H, L, d),), dtype=torch.uint8, device="cuda")
    rc = lib.entmax_attn_bwd_gqa(P(q), P(k), P(v), P(km), int(causal), window, P(tau), P(dout), P(ref[0]),
                                 P(ref[1]), P(ref[2]), B, H, hkv, L, d, dt, P(ws), ws.numel(), st)
    assert rc == 0, lib.entmax_attn_last_error()
    got = [torch.full_like(t, float("nan")) for t in ref]
    torch.cuda.synchronize()
    rc = lib.entmax_attn_bwd_noalloc(P(q), P(k), P(v), P(km), int(causal), window, P(tau), P(dout), P(got[0]),
                                     P(got[1]), P(got[2]), B, H, hkv, L, d, dt, st)
    assert rc == 0, lib.entmax_attn_last_error()
    torch.cuda.synchronize()
    for name, r, t in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(r, t), (name, float((r - t).abs().max()))


@pytest.mark.gpu
def test_noalloc_matches_workspace_backward(lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # first the long-context shape (B=1, H=32, L=8192, d=128: the wide
    # kernels and the fix-up pass), then a smaller padded bf16 case and a
    # grouped-query f32 case, each in the scratch the previous call left
    print("noalloc: long-context shape", flush=True)
    _both(lib, make_inputs("longctx"))
    print("noalloc: B=2 H=2 L=150 d=64 bf16, padded keys", flush=True)
    _both(lib, random_inputs(2, 2, 150, 64, "bf16", seed=21, key_lengths=[150, 97]))
    print("noalloc: B=1 H=4 H_kv=2 L=300 d=64 f32, causal window 32", flush=True)
    inp = random_inputs(1, 4, 300, 64, "f32", seed=22)
    inp["k"] = inp["k"][:, :2].contiguous()
    inp["v"] = inp["v"][:, :2].contiguous()
    _both(lib, inp, causal=True, window=32)
