"""ctypes binding of libentmax_attn.so: argument marshalling only.

Every function here checks the shape, dtype, device and contiguity of every
tensor it passes on (inputs, and outputs or workspaces the caller provides,
which are checked before anything is launched), allocates outputs with torch
when the caller gives none, and calls the C ABI declared in
``include/entmax_attn.h`` with raw device pointers and torch's current HIP
stream.  No step of the computation runs in Python, and there is no CPU
fallback: without the built library every call raises.
"""

import ctypes
import os

import torch

LIB_NAME = "libentmax_attn.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

ENTMAX_F32 = 0
ENTMAX_BF16 = 1

EXPORTS = (
    "entmax15_rows_bwd",
    "entmax15_rows_fwd",
    "entmax_attn_bwd",
    "entmax_attn_bwd_gqa",
    "entmax_attn_bwd_noalloc",
    "entmax_attn_bwd_saved",
    "entmax_attn_bwd_workspace_bytes",
    "entmax_attn_decode",
    "entmax_attn_decode_bwd",
    "entmax_attn_decode_bwd_workspace_size",
    "entmax_attn_decode_workspace_size",
    "entmax_attn_fwd",
    "entmax_attn_fwd_gqa",
    "entmax_attn_fwd_save",
    "entmax_attn_last_error",
    "entmax_attn_probs",
    "entmax_attn_probs_gqa",
    "entmax_attn_saved_bytes",
    "entmax_attn_status_string",
    "entmax_attn_version",
    "entmax_bisect_rows_bwd",
    "entmax_bisect_rows_fwd",
)

_lib = None


class EntmaxError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, code, message):
        super().__init__(message)
        self.code = code


def load_library(path=LIB_PATH):
    """Load the shared library (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{LIB_NAME} is not built ({path}); run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    vp, i32, u8p, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    lib.entmax_attn_fwd.argtypes = [vp, vp, vp, u8p, i32, i32, fp, fp, i32, i32, i32, i32, i32, vp]
    lib.entmax_attn_fwd.restype = i32
    sz = ctypes.c_size_t
    lib.entmax_attn_bwd.argtypes = [vp, vp, vp, u8p, i32, i32, fp, vp, fp, fp, fp, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.entmax_attn_bwd.restype = i32
    lib.entmax_attn_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.entmax_attn_bwd_workspace_bytes.restype = sz
    lib.entmax_attn_probs.argtypes = [vp, vp, u8p, i32, i32, fp, fp, i32, i32, i32, i32, i32, vp]
    lib.entmax_attn_probs.restype = i32
    # grouped-query variants: H_kv after H
    lib.entmax_attn_fwd_gqa.argtypes = [vp, vp, vp, u8p, i32, i32, fp, fp, i32, i32, i32, i32, i32, i32, vp]
    lib.entmax_attn_fwd_gqa.restype = i32
    lib.entmax_attn_bwd_gqa.argtypes = [vp, vp, vp, u8p, i32, i32, fp, vp, fp, fp, fp, i32, i32, i32, i32, i32, i32,
                                        vp, sz, vp]
    lib.entmax_attn_bwd_gqa.restype = i32
    lib.entmax_attn_bwd_noalloc.argtypes = [vp, vp, vp, u8p, i32, i32, fp, vp, fp, fp, fp, i32, i32, i32, i32, i32,
                                            i32, vp]
    lib.entmax_attn_bwd_noalloc.restype = i32
    lib.entmax_attn_probs_gqa.argtypes = [vp, vp, u8p, i32, i32, fp, fp, i32, i32, i32, i32, i32, i32, vp]
    lib.entmax_attn_probs_gqa.restype = i32
    lib.entmax_attn_saved_bytes.argtypes = [i32, i32, i32, i32]
    lib.entmax_attn_saved_bytes.restype = sz
    lib.entmax_attn_fwd_save.argtypes = [vp, vp, vp, u8p, i32, i32, fp, fp, vp, sz, i32, i32, i32, i32, i32, i32, vp]
    lib.entmax_attn_fwd_save.restype = i32
    lib.entmax_attn_bwd_saved.argtypes = [vp, vp, vp, u8p, i32, i32, fp, vp, vp, sz, fp, fp, fp, i32, i32, i32, i32,
                                          i32, i32, vp, sz, vp]
    lib.entmax_attn_bwd_saved.restype = i32
    lib.entmax15_rows_fwd.argtypes = [vp, u8p, fp, fp, i32, i32, i32, vp]
    lib.entmax15_rows_fwd.restype = i32
    lib.entmax15_rows_bwd.argtypes = [fp, fp, fp, i32, i32, vp]
    lib.entmax15_rows_bwd.restype = i32
    f32 = ctypes.c_float
    lib.entmax_bisect_rows_fwd.argtypes = [vp, u8p, fp, fp, i32, i32, f32, i32, vp]
    lib.entmax_bisect_rows_fwd.restype = i32
    lib.entmax_bisect_rows_bwd.argtypes = [fp, fp, fp, i32, i32, f32, vp]
    lib.entmax_bisect_rows_bwd.restype = i32
    lib.entmax_attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.entmax_attn_decode_workspace_size.restype = sz
    lib.entmax_attn_decode.argtypes = [vp, vp, vp, vp, i32, i32, fp, fp, vp, sz, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.entmax_attn_decode.restype = i32
    lib.entmax_attn_decode_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.entmax_attn_decode_bwd_workspace_size.restype = sz
    lib.entmax_attn_decode_bwd.argtypes = [vp, vp, vp, vp, i32, i32, fp, vp, fp, fp, fp, vp, sz, i32, i32, i32, i32,
                                           i32, i32, i32, vp]
    lib.entmax_attn_decode_bwd.restype = i32
    lib.entmax_attn_status_string.argtypes = [i32]
    lib.entmax_attn_status_string.restype = ctypes.c_char_p
    lib.entmax_attn_last_error.argtypes = []
    lib.entmax_attn_last_error.restype = ctypes.c_char_p
    lib.entmax_attn_version.argtypes = []
    lib.entmax_attn_version.restype = i32
    _lib = lib
    return lib


def _check(lib, rc):
    if rc != 0:
        status = lib.entmax_attn_status_string(rc).decode()
        msg = lib.entmax_attn_last_error().decode()
        raise EntmaxError(rc, f"{status}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.float32:
        return ENTMAX_F32
    if t.dtype == torch.bfloat16:
        return ENTMAX_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _check_qkv(q, k, v=None):
    """q [B, H, L, d]; k, v [B, H_kv, L, d] with H_kv dividing H. Returns H_kv."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d]")
    B, H, L, d = q.shape
    hkv = k.shape[1] if k.dim() == 4 else -1
    if hkv <= 0 or H % hkv != 0:
        raise ValueError("k must be [B, H_kv, L, d] with H_kv dividing H")
    for name, t in (("k", k), ("v", v)):
        if t is None:
            continue
        if t.shape != (B, hkv, L, d) or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must be [B, H_kv, L, d] with q's dtype and device")
    for t in (q, k, v):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("q, k, v must be contiguous GPU tensors")
    return hkv


def _check_mask(key_mask, q):
    if key_mask is None:
        return None
    B, _, L, _ = q.shape
    if key_mask.shape != (B, L) or key_mask.dtype != torch.uint8 or key_mask.device != q.device:
        raise ValueError("key_mask must be a [B, L] uint8 tensor on q's device")
    return key_mask.contiguous()


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _out(t, shape, like, name, dtype=torch.float32):
    """A caller-provided output (or auxiliary input) tensor: exactly ``shape``
    and ``dtype``, contiguous, on ``like``'s device; or None.  Raises
    ValueError before anything is launched."""
    if t is None:
        return None
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != like.device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {tuple(shape)} {dtype} tensor on {like.device} "
                         f"(got {tuple(t.shape)} {t.dtype} on {t.device})")
    return t


def _workspace(ws, need, like, name="workspace"):
    """A caller-provided workspace: a contiguous uint8 tensor of at least
    ``need`` bytes on ``like``'s device, or None to allocate one."""
    if ws is None:
        return torch.empty((max(need, 1),), dtype=torch.uint8, device=like.device)
    if ws.dtype != torch.uint8 or ws.device != like.device or not ws.is_contiguous() or ws.numel() < need:
        raise ValueError(f"{name} must be a contiguous uint8 tensor of at least {need} bytes on {like.device}")
    return ws


def entmax_attn_fwd(q, k, v, key_mask=None, causal=False, window=0, out=None, tau_out=None, want_tau=True):
    """O = entmax_1.5(Q K^T / sqrt(d)) V and the row thresholds tau.

    Returns (out [B, H, L, d] float32, tau [B, H, L] float32 or None).
    """
    lib = load_library()
    hkv = _check_qkv(q, k, v)
    km = _check_mask(key_mask, q)
    B, H, L, d = q.shape
    out = _out(out, (B, H, L, d), q, "out")
    tau_out = _out(tau_out, (B, H, L), q, "tau_out")
    if out is None:
        out = torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
    if tau_out is None and want_tau:
        tau_out = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    rc = lib.entmax_attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(km), int(bool(causal)), int(window),
                                 _ptr(out), _ptr(tau_out), B, H, hkv, L, d, _dtype_code(q), _stream(q))
    _check(lib, rc)
    return out, tau_out


def saved_bytes(B, H, L, d):
    """Bytes of device memory ``entmax_attn_fwd_save`` keeps the support in
    (a count and d/2 entries per query row)."""
    return int(load_library().entmax_attn_saved_bytes(B, H, L, d))


def entmax_attn_fwd_save(q, k, v, key_mask=None, causal=False, window=0, out=None, tau_out=None, saved=None):
    """``entmax_attn_fwd`` that also keeps each query row's support for
    ``entmax_attn_bwd_saved`` (spans above 2048 keys; elsewhere the buffer is
    not touched and the backward recomputes as usual).

    saved: a uint8 GPU tensor of at least ``saved_bytes`` bytes, or None to
    allocate one.  Returns (out, tau, saved)."""
    lib = load_library()
    hkv = _check_qkv(q, k, v)
    km = _check_mask(key_mask, q)
    B, H, L, d = q.shape
    out = _out(out, (B, H, L, d), q, "out")
    tau_out = _out(tau_out, (B, H, L), q, "tau_out")
    if out is None:
        out = torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
    if tau_out is None:
        tau_out = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    saved = _workspace(saved, saved_bytes(B, H, L, d), q, "saved")
    rc = lib.entmax_attn_fwd_save(_ptr(q), _ptr(k), _ptr(v), _ptr(km), int(bool(causal)), int(window),
                                  _ptr(out), _ptr(tau_out), _ptr(saved), saved.numel(), B, H, hkv, L, d,
                                  _dtype_code(q), _stream(q))
    _check(lib, rc)
    return out, tau_out, saved


def entmax_attn_bwd_saved(q, k, v, tau, dout, saved, key_mask=None, causal=False, window=0, dq=None, dk=None,
                          dv=None, workspace=None):
    """``entmax_attn_bwd`` on the support kept by ``entmax_attn_fwd_save``
    (same inputs and masks): the query side reads each row's support instead
    of recomputing the scores.  Returns (dq, dk, dv)."""
    lib = load_library()
    hkv = _check_qkv(q, k, v)
    _check_qkv(q, dout)
    if dout.shape != q.shape:
        raise ValueError("dout must match q")
    km = _check_mask(key_mask, q)
    B, H, L, d = q.shape
    if tau is None or saved is None:
        raise ValueError("tau and saved are required")
    _out(tau, (B, H, L), q, "tau")
    saved = _workspace(saved, saved_bytes(B, H, L, d), q, "saved")
    dq = _out(dq, (B, H, L, d), q, "dq")
    dk = _out(dk, (B, hkv, L, d), q, "dk")
    dv = _out(dv, (B, hkv, L, d), q, "dv")
    workspace = _workspace(workspace, bwd_workspace_bytes(B, H, L, d), q)
    mk = lambda h: torch.empty((B, h, L, d), dtype=torch.float32, device=q.device)  # noqa: E731
    dq = mk(H) if dq is None else dq
    dk = mk(hkv) if dk is None else dk
    dv = mk(hkv) if dv is None else dv
    rc = lib.entmax_attn_bwd_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(km), int(bool(causal)), int(window), _ptr(tau),
                                   _ptr(dout), _ptr(saved), saved.numel(), _ptr(dq), _ptr(dk), _ptr(dv), B, H, hkv,
                                   L, d, _dtype_code(q), _ptr(workspace), workspace.numel(), _stream(q))
    _check(lib, rc)
    return dq, dk, dv


def bwd_workspace_bytes(B, H, L, d):
    """Bytes of device workspace ``entmax_attn_bwd`` needs (c_i per query row)."""
    return int(load_library().entmax_attn_bwd_workspace_bytes(B, H, L, d))


def entmax_attn_bwd(q, k, v, tau, dout, key_mask=None, causal=False, window=0, dq=None, dk=None, dv=None,
                    workspace=None):
    """Gradients float32: dq [B, H, L, d], dk and dv [B, H_kv, L, d], from the forward's tau.

    workspace: a uint8 GPU tensor of at least ``bwd_workspace_bytes`` bytes,
    or None to allocate one.  Deterministic (no atomics)."""
    lib = load_library()
    hkv = _check_qkv(q, k, v)
    _check_qkv(q, dout)
    if dout.shape != q.shape:
        raise ValueError("dout must match q")
    km = _check_mask(key_mask, q)
    B, H, L, d = q.shape
    if tau is None:
        raise ValueError("tau is required")
    _out(tau, (B, H, L), q, "tau")
    dq = _out(dq, (B, H, L, d), q, "dq")
    dk = _out(dk, (B, hkv, L, d), q, "dk")
    dv = _out(dv, (B, hkv, L, d), q, "dv")
    need = bwd_workspace_bytes(B, H, L, d)
    workspace = _workspace(workspace, need, q)
    mk = lambda h: torch.empty((B, h, L, d), dtype=torch.float32, device=q.device)  # noqa: E731
    dq = mk(H) if dq is None else dq
    dk = mk(hkv) if dk is None else dk
    dv = mk(hkv) if dv is None else dv
    rc = lib.entmax_attn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(km), int(bool(causal)), int(window), _ptr(tau),
                                 _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, H, hkv, L, d, _dtype_code(q),
                                 _ptr(workspace), workspace.numel(), _stream(q))
    _check(lib, rc)
    return dq, dk, dv


def entmax_attn_bwd_noalloc(q, k, v, tau, dout, dq, dk, dv, key_mask=None, causal=False, window=0):
    """``entmax_attn_bwd`` into caller-provided dq, dk, dv with no allocation:
    c_i lives in the library's built-in scratch (at most 1048576 query rows
    B H L; calls in flight at once on one GPU race).  Returns (dq, dk, dv)."""
    lib = load_library()
    hkv = _check_qkv(q, k, v)
    _check_qkv(q, dout)
    if dout.shape != q.shape:
        raise ValueError("dout must match q")
    km = _check_mask(key_mask, q)
    B, H, L, d = q.shape
    if tau is None or dq is None or dk is None or dv is None:
        raise ValueError("tau, dq, dk and dv are required (this call allocates nothing)")
    _out(tau, (B, H, L), q, "tau")
    _out(dq, (B, H, L, d), q, "dq")
    _out(dk, (B, hkv, L, d), q, "dk")
    _out(dv, (B, hkv, L, d), q, "dv")
    rc = lib.entmax_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(km), int(bool(causal)), int(window), _ptr(tau),
                                     _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, H, hkv, L, d, _dtype_code(q),
                                     _stream(q))
    _check(lib, rc)
    return dq, dk, dv


def entmax_attn_probs(q, k, tau, key_mask=None, causal=False, window=0, probs=None):
    """Dense attention weights [B, H, L, L] float32 recomputed from tau."""
    lib = load_library()
    hkv = _check_qkv(q, k)
    km = _check_mask(key_mask, q)
    B, H, L, d = q.shape
    if tau is None:
        raise ValueError("tau is required")
    _out(tau, (B, H, L), q, "tau")
    probs = _out(probs, (B, H, L, L), q, "probs")
    if probs is None:
        probs = torch.empty((B, H, L, L), dtype=torch.float32, device=q.device)
    rc = lib.entmax_attn_probs_gqa(_ptr(q), _ptr(k), _ptr(km), int(bool(causal)), int(window), _ptr(tau),
                                   _ptr(probs), B, H, hkv, L, d, _dtype_code(q), _stream(q))
    _check(lib, rc)
    return probs


def decode_workspace_bytes(B, H, H_kv, S, d, window=0, Lq=1):
    """Bytes of device workspace ``entmax_attn_decode`` needs."""
    return int(load_library().entmax_attn_decode_workspace_size(B, H, H_kv, Lq, S, d, int(window)))


def entmax_attn_decode(q, k_cache, v_cache, seqlens, window=0, out=None, tau=None, workspace=None,
                       want_tau=True, causal=True):
    """Decode-time 1.5-entmax attention: the newest queries of each sequence
    against a key/value cache.

    q [B, H, d] (one new token) or [B, H, Lq, d]; k_cache, v_cache
    [B, H_kv, S, d] (same dtype, float32 or bfloat16); seqlens [B] int32 on
    the GPU (valid cache positions per sequence, the new tokens' included:
    query i sits at seqlens[b] - Lq + i); window 0 (every earlier key) or
    W > 0.  causal=False: every query attends all seqlens[b] keys (window 0).  workspace: a uint8 GPU tensor of at least
    ``decode_workspace_bytes`` bytes, or None to allocate one.  Returns
    (out float32 shaped like q, tau float32 shaped like q without d, or None).
    """
    lib = load_library()
    if q.dim() not in (3, 4) or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B, H, d] or [B, H, Lq, d]; k_cache and v_cache [B, H_kv, S, d] of one shape")
    B, H, d = q.shape[0], q.shape[1], q.shape[-1]
    Lq = 1 if q.dim() == 3 else q.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != d or H % k_cache.shape[1] != 0:
        raise ValueError("k_cache must be [B, H_kv, S, d] with H_kv dividing H")
    for name, x in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not x.is_cuda or not x.is_contiguous() or x.dtype != q.dtype:
            raise ValueError(f"{name} must be a contiguous GPU tensor of q's dtype")
    if seqlens.shape != (B,) or seqlens.dtype != torch.int32 or seqlens.device != q.device:
        raise ValueError("seqlens must be a [B] int32 tensor on q's device")
    hkv, S = k_cache.shape[1], k_cache.shape[2]
    need = decode_workspace_bytes(B, H, hkv, S, d, window, Lq)
    workspace = _workspace(workspace, need, q)
    out = _out(out, tuple(q.shape), q, "out")
    tau = _out(tau, tuple(q.shape[:-1]), q, "tau")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if tau is None and want_tau:
        tau = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    rc = lib.entmax_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens.contiguous()),
                                int(bool(causal)), int(window),
                                _ptr(out), _ptr(tau), _ptr(workspace), workspace.numel(),
                                B, H, hkv, Lq, S, d, _dtype_code(q), _stream(q))
    _check(lib, rc)
    return out, tau


def decode_bwd_workspace_bytes(B, H, H_kv, S, d, window=0, Lq=1):
    """Bytes of device workspace ``entmax_attn_decode_bwd`` needs."""
    return int(load_library().entmax_attn_decode_bwd_workspace_size(B, H, H_kv, Lq, S, d, int(window)))


def entmax_attn_decode_bwd(q, k_cache, v_cache, seqlens, tau, dout, window=0, causal=True, dq=None, dk=None,
                           dv=None, workspace=None):
    """Gradients of ``entmax_attn_decode`` from its tau: (dq float32 shaped
    like q, dk and dv float32 [B, H_kv, S, d]).  Arguments as for the
    forward, plus tau (the forward's) and dout shaped like q.  workspace: a
    uint8 GPU tensor of at least ``decode_bwd_workspace_bytes`` bytes, or
    None to allocate one.  Deterministic (no atomics)."""
    lib = load_library()
    if q.dim() not in (3, 4) or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B, H, d] or [B, H, Lq, d]; k_cache and v_cache [B, H_kv, S, d] of one shape")
    B, H, d = q.shape[0], q.shape[1], q.shape[-1]
    Lq = 1 if q.dim() == 3 else q.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != d or H % k_cache.shape[1] != 0:
        raise ValueError("k_cache must be [B, H_kv, S, d] with H_kv dividing H")
    for name, x in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("dout", dout)):
        if not x.is_cuda or not x.is_contiguous() or x.dtype != q.dtype:
            raise ValueError(f"{name} must be a contiguous GPU tensor of q's dtype")
    if dout.shape != q.shape:
        raise ValueError("dout must match q")
    if seqlens.shape != (B,) or seqlens.dtype != torch.int32 or seqlens.device != q.device:
        raise ValueError("seqlens must be a [B] int32 tensor on q's device")
    if tau is None:
        raise ValueError("tau is required")
    _out(tau, tuple(q.shape[:-1]), q, "tau")
    hkv, S = k_cache.shape[1], k_cache.shape[2]
    dq = _out(dq, tuple(q.shape), q, "dq")
    dk = _out(dk, (B, hkv, S, d), q, "dk")
    dv = _out(dv, (B, hkv, S, d), q, "dv")
    need = decode_bwd_workspace_bytes(B, H, hkv, S, d, window, Lq)
    workspace = _workspace(workspace, need, q)
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty((B, hkv, S, d), dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty((B, hkv, S, d), dtype=torch.float32, device=q.device)
    rc = lib.entmax_attn_decode_bwd(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens.contiguous()),
                                    int(bool(causal)), int(window), _ptr(tau), _ptr(dout), _ptr(dq), _ptr(dk),
                                    _ptr(dv), _ptr(workspace), workspace.numel(), B, H, hkv, Lq, S, d,
                                    _dtype_code(q), _stream(q))
    _check(lib, rc)
    return dq, dk, dv


def entmax_bisect_rows(scores, alpha=1.5, mask=None, p=None, tau=None, want_tau=True):
    """Row-wise alpha-entmax (alpha in (1, 2]) of a [R, L] score matrix
    (float32 or bfloat16).

    mask: [R, L] uint8 (nonzero = allowed) or None.  Returns
    (p [R, L] float32, tau [R] float32 in score units or None), with
    p = [(alpha - 1)(s - tau)]_+^(1/(alpha - 1)).
    """
    lib = load_library()
    if scores.dim() != 2 or not scores.is_cuda or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous [R, L] GPU tensor")
    R, L = scores.shape
    if mask is not None:
        if mask.shape != (R, L) or mask.dtype != torch.uint8 or mask.device != scores.device:
            raise ValueError("mask must be a [R, L] uint8 tensor on the scores' device")
        mask = mask.contiguous()
    p = _out(p, (R, L), scores, "p")
    tau = _out(tau, (R,), scores, "tau")
    if p is None:
        p = torch.empty((R, L), dtype=torch.float32, device=scores.device)
    if tau is None and want_tau:
        tau = torch.empty((R,), dtype=torch.float32, device=scores.device)
    rc = lib.entmax_bisect_rows_fwd(_ptr(scores), _ptr(mask), _ptr(p), _ptr(tau), R, L, float(alpha),
                                    _dtype_code(scores), _stream(scores))
    _check(lib, rc)
    return p, tau


def entmax_bisect_rows_bwd(p, dp, alpha=1.5, ds=None):
    """Gradient of the scores of ``entmax_bisect_rows`` from the gradient of p
    (float32 [R, L]); alpha must be the forward's."""
    lib = load_library()
    for name, t in (("p", p), ("dp", dp)):
        if t.dim() != 2 or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [R, L] float32 GPU tensor")
    if dp.shape != p.shape or dp.device != p.device:
        raise ValueError("dp must match p (shape and device)")
    R, L = p.shape
    ds = _out(ds, (R, L), p, "ds")
    if ds is None:
        ds = torch.empty((R, L), dtype=torch.float32, device=p.device)
    rc = lib.entmax_bisect_rows_bwd(_ptr(p), _ptr(dp), _ptr(ds), R, L, float(alpha), _stream(p))
    _check(lib, rc)
    return ds


def entmax15_rows(scores, mask=None, p=None, tau=None, want_tau=True):
    """Row-wise 1.5-entmax of a [R, L] score matrix (float32 or bfloat16).

    mask: [R, L] uint8 (nonzero = allowed) or None.  Returns
    (p [R, L] float32, tau [R] float32 in score units or None).
    """
    lib = load_library()
    if scores.dim() != 2 or not scores.is_cuda or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous [R, L] GPU tensor")
    R, L = scores.shape
    if mask is not None:
        if mask.shape != (R, L) or mask.dtype != torch.uint8 or mask.device != scores.device:
            raise ValueError("mask must be a [R, L] uint8 tensor on the scores' device")
        mask = mask.contiguous()
    p = _out(p, (R, L), scores, "p")
    tau = _out(tau, (R,), scores, "tau")
    if p is None:
        p = torch.empty((R, L), dtype=torch.float32, device=scores.device)
    if tau is None and want_tau:
        tau = torch.empty((R,), dtype=torch.float32, device=scores.device)
    rc = lib.entmax15_rows_fwd(_ptr(scores), _ptr(mask), _ptr(p), _ptr(tau), R, L, _dtype_code(scores),
                               _stream(scores))
    _check(lib, rc)
    return p, tau


def entmax15_rows_bwd(p, dp, ds=None):
    """Gradient of the scores of ``entmax15_rows`` from the gradient of p (float32 [R, L])."""
    lib = load_library()
    for name, t in (("p", p), ("dp", dp)):
        if t.dim() != 2 or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [R, L] float32 GPU tensor")
    if dp.shape != p.shape or dp.device != p.device:
        raise ValueError("dp must match p (shape and device)")
    R, L = p.shape
    ds = _out(ds, (R, L), p, "ds")
    if ds is None:
        ds = torch.empty((R, L), dtype=torch.float32, device=p.device)
    rc = lib.entmax15_rows_bwd(_ptr(p), _ptr(dp), _ptr(ds), R, L, _stream(p))
    _check(lib, rc)
    return ds


def raw_call(name, *args):
    """Call an exported symbol with raw ctypes arguments; returns its result.

    For tests of the boundary itself (error codes on bad arguments)."""
    lib = load_library()
    return getattr(lib, name)(*args)
