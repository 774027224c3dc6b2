"""CPU tests of the C-ABI boundary: the library loads, exports every symbol
the header declares, and rejects bad arguments with the documented status
codes before touching the GPU (argument checks run before any HIP call)."""

import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b(entmax\w+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from entmax_amd import load_library
    return load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("entmax_attn_fwd", "entmax_attn_bwd", "entmax_attn_probs"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from entmax_amd import LIB_PATH, EXPORTS
    declared = _declared_functions()
    dyn = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\w+)$", dyn, flags=re.M))
    for n in declared:
        assert n in exported, n
        assert hasattr(lib, n), n
    assert sorted(EXPORTS) == declared


def test_status_strings(lib):
    assert lib.entmax_attn_status_string(0) == b"ok"
    assert lib.entmax_attn_status_string(1) == b"invalid argument"
    assert lib.entmax_attn_status_string(2) == b"unsupported configuration"
    assert lib.entmax_attn_status_string(3) == b"HIP error"
    assert lib.entmax_attn_version() == 2


P = ctypes.c_void_p(16)   # never dereferenced: every call below is rejected first


def _fwd(lib, q=P, k=P, v=P, mask=None, causal=0, window=0, out=P, tau=None, B=1, H=1, L=8, d=64, dtype=1):
    return lib.entmax_attn_fwd(q, k, v, mask, causal, window, out, tau, B, H, L, d, dtype, None)


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, 1), ({"k": None}, 1), ({"v": None}, 1), ({"out": None}, 1),
    ({"B": 0}, 1), ({"H": -1}, 1), ({"L": 0}, 1),
    ({"window": -1, "causal": 1}, 1), ({"window": 32, "causal": 0}, 1),
    ({"d": 96}, 2), ({"d": 256}, 2), ({"dtype": 7}, 2), ({"L": 65537}, 2),
])
def test_fwd_rejects_bad_arguments(lib, kw, code):
    assert _fwd(lib, **kw) == code
    assert lib.entmax_attn_last_error() != b""


W256 = ctypes.c_void_p(256)   # a 256-byte aligned stand-in for a workspace


def _bwd_args(lib, B=1, H=1, L=8, d=64):
    # q, k, v, mask, causal, window, tau, dout, dq, dk, dv, B, H, L, d, dtype, ws, ws_bytes, stream
    ws = lib.entmax_attn_bwd_workspace_bytes(B, H, L, d)
    return [P, P, P, None, 0, 0, P, P, P, P, P, B, H, L, d, 1, W256, ws, None]


def test_bwd_workspace_size(lib):
    # c_i of every query row and a bucket counter per row, each rounded up
    # to 256 bytes, then 256 bytes for the overflow flag
    assert lib.entmax_attn_bwd_workspace_bytes(1, 32, 8192, 128) == 2 * 32 * 8192 * 4 + 256
    assert lib.entmax_attn_bwd_workspace_bytes(2, 3, 7, 64) == 3 * 256
    assert lib.entmax_attn_bwd_workspace_bytes(0, 3, 7, 64) == 0
    assert lib.entmax_attn_bwd_workspace_bytes(1, 1, -1, 64) == 0


def test_bwd_and_probs_reject_null(lib):
    args = _bwd_args(lib)
    for i in (0, 1, 2, 6, 7, 8, 9, 10, 16):
        a = list(args)
        a[i] = None
        assert lib.entmax_attn_bwd(*a) == 1, i
    assert lib.entmax_attn_bwd(*args[:4], 0, 5, *args[6:]) == 1         # window without causal
    a = list(args)
    a[17] = args[17] - 1                                                 # workspace too small
    assert lib.entmax_attn_bwd(*a) == 1
    assert b"workspace" in lib.entmax_attn_last_error()
    a = list(args)
    a[16] = ctypes.c_void_p(272)                                         # workspace not 256-byte aligned
    assert lib.entmax_attn_bwd(*a) == 1
    assert lib.entmax_attn_probs(P, P, None, 0, 0, None, P, 1, 1, 8, 64, 1, None) == 1
    assert lib.entmax_attn_probs(P, P, None, 0, 0, P, P, 1, 1, 8, 32, 1, None) == 2


def test_saved_support_size_and_arguments(lib):
    # a count per query row (rounded up to 256 bytes), then d/2 entries of
    # 8 bytes per row
    assert lib.entmax_attn_saved_bytes(1, 32, 8192, 128) == 32 * 8192 * 4 + 32 * 8192 * 64 * 8
    assert lib.entmax_attn_saved_bytes(2, 3, 7, 64) == 256 + 42 * 32 * 8
    assert lib.entmax_attn_saved_bytes(0, 3, 7, 64) == 0
    sb = lib.entmax_attn_saved_bytes(1, 1, 8, 64)
    # q, k, v, mask, causal, window, out, tau, saved, saved_bytes, B, H, Hkv, L, d, dtype, stream
    fargs = [P, P, P, None, 0, 0, P, P, W256, sb, 1, 1, 1, 8, 64, 1, None]
    for i in (0, 1, 2, 6, 7, 8):
        a = list(fargs)
        a[i] = None
        assert lib.entmax_attn_fwd_save(*a) == 1, i
    a = list(fargs)
    a[9] = sb - 1                                                        # saved buffer too small
    assert lib.entmax_attn_fwd_save(*a) == 1
    assert b"saved" in lib.entmax_attn_last_error()
    a = list(fargs)
    a[8] = ctypes.c_void_p(272)                                          # not 256-byte aligned
    assert lib.entmax_attn_fwd_save(*a) == 1
    ws = lib.entmax_attn_bwd_workspace_bytes(1, 1, 8, 64)
    # q, k, v, mask, causal, window, tau, dout, saved, saved_bytes, dq, dk, dv, B, H, Hkv, L, d, dtype, ws,
    # ws_bytes, stream
    bargs = [P, P, P, None, 0, 0, P, P, W256, sb, P, P, P, 1, 1, 1, 8, 64, 1, W256, ws, None]
    for i in (0, 1, 2, 6, 7, 8, 10, 11, 12, 19):
        a = list(bargs)
        a[i] = None
        assert lib.entmax_attn_bwd_saved(*a) == 1, i
    a = list(bargs)
    a[9] = sb - 1
    assert lib.entmax_attn_bwd_saved(*a) == 1
    a = list(bargs)
    a[20] = ws - 1
    assert lib.entmax_attn_bwd_saved(*a) == 1
    a = list(bargs)
    a[17] = 96                                                           # unsupported d
    assert lib.entmax_attn_bwd_saved(*a) == 2


def test_binding_validates_before_calling():
    import torch
    from entmax_amd import entmax_attn_fwd
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        entmax_attn_fwd(q, q, q)          # CPU tensors are refused by the binding
    with pytest.raises(TypeError):
        from entmax_amd._binding import _dtype_code
        _dtype_code(torch.zeros(1, dtype=torch.float16))


def test_binding_validates_outputs_before_calling():
    # caller-provided outputs and workspaces of the wrong shape, dtype,
    # device or layout are refused by the binding, before any launch
    import torch
    from entmax_amd._binding import _out, _workspace
    like = torch.zeros(2, 3, 8, 64)
    good = torch.zeros(2, 3, 8, 64)
    assert _out(good, (2, 3, 8, 64), like, "out") is good
    assert _out(None, (2, 3, 8, 64), like, "out") is None
    for bad in (torch.zeros(2, 3, 8, 32), torch.zeros(2, 3, 8, 64, dtype=torch.bfloat16),
                torch.zeros(2, 3, 64, 8).transpose(2, 3)):
        with pytest.raises(ValueError):
            _out(bad, (2, 3, 8, 64), like, "out")
    assert _workspace(torch.zeros(300, dtype=torch.uint8), 256, like).numel() == 300
    for bad in (torch.zeros(100, dtype=torch.uint8), torch.zeros(300, dtype=torch.float32)):
        with pytest.raises(ValueError):
            _workspace(bad, 256, like)


def test_grouped_query_rejects_bad_kv_heads(lib):
    # H_kv must divide H
    for hkv in (0, -1, 3):
        assert lib.entmax_attn_fwd_gqa(P, P, P, None, 0, 0, P, None, 1, 4, hkv, 8, 64, 1, None) == 1
        assert lib.entmax_attn_bwd_gqa(P, P, P, None, 0, 0, P, P, P, P, P, 1, 4, hkv, 8, 64, 1, W256, 1 << 20,
                                       None) == 1
        assert lib.entmax_attn_probs_gqa(P, P, None, 0, 0, P, P, 1, 4, hkv, 8, 64, 1, None) == 1
    assert b"H_kv" in lib.entmax_attn_last_error()


def test_binding_checks_grouped_shapes():
    import torch
    from entmax_amd._binding import _check_qkv
    q = torch.zeros(1, 4, 8, 64)
    with pytest.raises(ValueError):
        _check_qkv(q, torch.zeros(1, 3, 8, 64))     # 3 does not divide 4
    with pytest.raises(ValueError):
        _check_qkv(q, torch.zeros(1, 2, 8, 64), torch.zeros(1, 4, 8, 64))   # v must match k


def test_rows_reject_bad_arguments(lib):
    # alpha outside (1, 2], null pointers, L not a multiple of 4
    for a in (1.0, 0.9, 2.01, float("nan")):
        assert lib.entmax_bisect_rows_fwd(P, None, P, None, 4, 8, a, 0, None) == 1
        assert lib.entmax_bisect_rows_bwd(P, P, P, 4, 8, a, None) == 1
    assert b"alpha" in lib.entmax_attn_last_error()
    assert lib.entmax_bisect_rows_fwd(None, None, P, None, 4, 8, 1.5, 0, None) == 1
    assert lib.entmax_bisect_rows_fwd(P, None, P, None, 4, 10, 1.5, 0, None) == 2
    assert lib.entmax_bisect_rows_fwd(P, None, P, None, 4, 8, 1.5, 5, None) == 2
    assert lib.entmax15_rows_fwd(P, None, P, None, 0, 8, 0, None) == 1
    assert lib.entmax15_rows_bwd(P, None, P, 4, 8, None) == 1


def test_decode_rejects_bad_arguments(lib):
    ws = lib.entmax_attn_decode_workspace_size(2, 4, 4, 1, 64, 64, 0)
    assert ws > 0 and ws % 256 == 0
    assert lib.entmax_attn_decode_workspace_size(0, 4, 4, 1, 64, 64, 0) == 0
    assert lib.entmax_attn_decode_workspace_size(2, 4, 3, 1, 64, 64, 0) == 0
    assert lib.entmax_attn_decode_workspace_size(2, 4, 4, 0, 64, 64, 0) == 0
    W = ctypes.c_void_p(256)
    # q, k, v, seqlens, causal, window, out, tau, ws, ws_bytes, B, H, Hkv, Lq, S, d, dtype, stream
    ok = [P, P, P, P, 1, 0, P, None, W, ws, 2, 4, 4, 1, 64, 64, 1, None]
    for i in (0, 1, 2, 3, 6, 8):
        a = list(ok)
        a[i] = None
        assert lib.entmax_attn_decode(*a) == 1
    bad = {9: ws - 1, 12: 3, 5: -1, 13: 0, 15: 96, 16: 7}
    for i, val in bad.items():
        a = list(ok)
        a[i] = val
        assert lib.entmax_attn_decode(*a) == (2 if i in (15, 16) else 1), i
    a = list(ok)
    a[13] = 65           # Lq above S
    assert lib.entmax_attn_decode(*a) == 1
    a = list(ok)
    a[4], a[5] = 0, 8    # a window without causal
    assert lib.entmax_attn_decode(*a) == 1
    a = list(ok)
    a[8] = ctypes.c_void_p(272)      # not 256-byte aligned
    assert lib.entmax_attn_decode(*a) == 1


def test_entry_points_reject_misaligned_pointers(lib):
    # rows are read and written with 16-byte vector accesses; tau and probs
    # with 4-byte ones: a misaligned pointer is refused before any launch
    M16, M4 = ctypes.c_void_p(24), ctypes.c_void_p(18)
    for kw in ({"q": M16}, {"k": M16}, {"v": M16}, {"out": M16}, {"tau": M4}):
        assert _fwd(lib, **kw) == 1, kw
    assert b"aligned" in lib.entmax_attn_last_error()
    args = _bwd_args(lib)
    for i, bad in ((0, M16), (1, M16), (2, M16), (6, M4), (7, M16), (8, M16), (9, M16), (10, M16)):
        a = list(args)
        a[i] = bad
        assert lib.entmax_attn_bwd(*a) == 1, i
    assert lib.entmax_attn_probs(M16, P, None, 0, 0, P, P, 1, 1, 8, 64, 1, None) == 1
    assert lib.entmax_attn_probs(P, P, None, 0, 0, P, M4, 1, 1, 8, 64, 1, None) == 1
    assert lib.entmax_bisect_rows_fwd(M16, None, P, None, 4, 8, 1.5, 0, None) == 1
    assert lib.entmax_bisect_rows_fwd(P, M16, P, None, 4, 8, 1.5, 0, None) == 1
    assert lib.entmax_bisect_rows_fwd(P, None, P, M4, 4, 8, 1.5, 0, None) == 1
    assert lib.entmax_bisect_rows_bwd(P, P, M16, 4, 8, 1.5, None) == 1
    ws = lib.entmax_attn_decode_workspace_size(2, 4, 4, 1, 64, 64, 0)
    ok = [P, P, P, P, 1, 0, P, None, ctypes.c_void_p(256), ws, 2, 4, 4, 1, 64, 64, 1, None]
    for i, bad in ((0, M16), (1, M16), (2, M16), (3, M4), (6, M16), (7, M4)):
        a = list(ok)
        a[i] = bad
        assert lib.entmax_attn_decode(*a) == 1, i


def test_missing_library_fails_loudly(tmp_path):
    # no fallback of any kind: without the built library every call raises
    import subprocess
    import sys
    code = (
        "import entmax_amd._binding as b\n"
        "b._lib = None\n"
        "b.LIB_PATH = '" + str(tmp_path / "absent.so") + "'\n"
        "try:\n"
        "    b.load_library(b.LIB_PATH)\n"
        "except RuntimeError as e:\n"
        "    print('raised', e)\n"
    )
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "raised" in out.stdout and "not built" in out.stdout
