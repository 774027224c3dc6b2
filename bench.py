"""Throughput of 1.5-entmax attention on one MI355X, against its roofline.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|NAME]

By default (``--workload all``) one process times the five workloads of the
metric (tiny, encoder, long, decoder, longctx: L = 64 .. 8192) and prints ONE
JSON line headed by the largest single-GPU workload, ``longctx`` (B1 H32
L8192 d128 bf16, forward + backward); the other four are reported under
``configs``, each with its time, roofline fraction, measured traffic and
zero fraction.

One step = one pass of the whole path over one batch of synthetic input:
the forward (scores, masks, row max, tau by bisection, P, O = P V) for the
forward workloads, forward + backward for ``longctx``.  Inputs are already
resident in HBM when the timed region starts; the timed steps rotate over
enough copies of the input/output buffers (> 512 MB in total) that no step
is served from the 256 MB Infinity Cache.  Every workload gets W warmup
steps, then EXACTLY K timed steps between ``torch.cuda.synchronize()``
calls, with HIP events on the launch stream (torch's current stream, which
the binding hands to the library).

FLOP conventions (stated once, used everywhere):
  * effective (``value``): 4 d per allowed (query, key) pair for the forward
    (Q K^T and A V as dense products; zeros of A count as done) and 10 d
    per pair for the backward (S, dP, dQ, dK and dV as dense products);
  * algorithmic (``roofline``): the method's minimum work, 2 d per allowed
    pair (Q K^T) + 2 d per nonzero of A (A V) for the forward, and
    2 d per pair (S recomputed) + 8 d per nonzero (dP, dQ, dK, dV on the
    support) for the backward;
  * bytes (HBM-bound workloads): Q, K and V rows that some query may
    attend, O and tau in float32 and the key mask, each moved once.
``roofline`` describes the longest call of the headline step (its kernels
named), measured live with HIP events; ``traffic`` is the rocprofv3
FETCH_SIZE + WRITE_SIZE of that call's kernels per launch, copy-calibrated
(profiles/traffic.json), or null when the kernel sources changed since.
``cpu_baseline`` times the float64 oracle on the host cores before the GPU
is touched: a process pool of ``cores`` workers (one BLAS thread each) on a
bounded sample of the headline workload, plus the same sample's rate on one
worker.
"""

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "1.5-entmax attn fwd: effective TFLOP/s + % MFMA/HBM roofline, L=128..8192"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6
MFMA_F32_PEAK_TFLOPS = 157.3
MALL_BYTES = 256 * 2 ** 20
ORDER = ("tiny", "encoder", "long", "decoder", "longctx")
HEADLINE = "longctx"
BOUND = {"tiny": "hbm", "encoder": "hbm", "long": "mfma", "decoder": "hbm", "longctx": "mfma"}
FWD_EFF, BWD_EFF = 4, 10          # effective FLOPs per allowed pair, in units of d


def allowed_pairs_per_head(w, key_mask):
    """Number of allowed (query, key) pairs for each batch entry (list)."""
    import numpy as np
    L = w.L
    if key_mask is not None:
        lens = key_mask.sum(dim=1).tolist()
        return [L * int(n) for n in lens]
    if w.causal and w.window > 0:
        i = np.arange(L)
        n = int(np.minimum(i + 1, w.window).sum())
    elif w.causal:
        n = L * (L + 1) // 2
    else:
        n = L * L
    return [n] * w.B


def algorithmic_bytes(w, key_mask):
    """HBM bytes one forward launch must move at least: Q, K and V rows that
    some query may attend (valid keys only), O (fp32), tau (fp32), mask."""
    esz = 4 if w.dtype == "f32" else 2
    row = w.d * esz
    q = w.B * w.H * w.L * row
    if key_mask is not None:
        kv_rows = int(key_mask.sum().item()) * w.H
    else:
        kv_rows = w.B * w.H * w.L
    o = w.B * w.H * w.L * w.d * 4
    tau = w.B * w.H * w.L * 4
    mask = 0 if key_mask is None else w.B * w.L
    return q + 2 * kv_rows * row + o + tau + mask


def saved_bwd_bytes(w, nnz):
    """HBM bytes the backward on the saved support must move at least: Q, K,
    V and dO read once, tau and the support (a count per row, 8 bytes per
    entry) read, dQ, dK and dV written in fp32.  It forms no score, so it is
    priced against HBM, not the MFMA peak."""
    esz = 4 if w.dtype == "f32" else 2
    rows = w.B * w.H * w.L
    return 4 * rows * w.d * esz + 2 * rows * 4 + 8 * nnz + 3 * rows * w.d * 4


def kernel_source_sha():
    """SHA-256 over the HIP sources; measured counters are tied to it."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "entmax_amd", "csrc")
    for f in sorted(os.listdir(src)):
        with open(os.path.join(src, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel="fwd"):
    """HBM bytes per launch of the workload's forward (or backward) call,
    from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded in
    profiles/traffic.json, or None when none were taken for the current
    kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh).get(workload if kernel == "fwd" else f"{workload}_{kernel}")
    if not rec or rec.get("source_sha") != kernel_source_sha():
        return None
    return rec["traffic_bytes"]


def copy_probe(mib=256, reps=10):
    """A plain device copy of known size, for calibrating the byte counters."""
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "reps": reps}))


def copy_bandwidth(mib=1024, reps=10):
    """Read + write GB/s of a plain 1 GiB device-to-device copy (median of
    ``reps`` timed copies), the measured HBM ceiling beside the 8 TB/s spec."""
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    del src, dst
    return 2 * n * 4 / (statistics.median(ts) * 1e-3) / 1e9


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the host cores
# ---------------------------------------------------------------------------

_CPU_INPUTS = {}


def _cpu_task(task):
    """One oracle task in a worker: (workload, b, h, rows or None, part)."""
    from threadpoolctl import threadpool_limits
    from oracle import attention_backward, attention_forward
    name, b, h, rows, part = task
    inp = _CPU_INPUTS[name]
    w = inp["workload"]
    with threadpool_limits(limits=1):
        if part == "fwd":
            import numpy as np
            attention_forward(inp["q"], inp["k"], inp["v"], inp["key_mask"], w.causal, w.window,
                              heads=[(b, h)], rows=None if rows is None else np.arange(*rows))
        else:
            attention_backward(inp["q"], inp["k"], inp["v"], inp["dout"], inp["key_mask"], w.causal, w.window,
                               heads=[(b, h)])
    return task


def _cpu_tasks(name, n_heads):
    """Oracle tasks covering n_heads whole (b, h) slices of a workload and
    the effective FLOPs they stand for.  Long rows are split into blocks of
    1024 query rows for the forward (the oracle's backward already works in
    row blocks), which bounds each worker's memory."""
    from entmax_amd.workloads import WORKLOADS
    w = WORKLOADS[name]
    inp = _CPU_INPUTS[name]
    pairs = allowed_pairs_per_head(w, inp["key_mask"])
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:n_heads]
    tasks, flop = [], 0.0
    for (b, h) in heads:
        if w.L > 2048:
            tasks += [(name, b, h, (r0, min(w.L, r0 + 1024)), "fwd") for r0 in range(0, w.L, 1024)]
        else:
            tasks.append((name, b, h, None, "fwd"))
        flop += FWD_EFF * w.d * pairs[b]
        if w.backward:
            tasks.append((name, b, h, None, "bwd"))
            flop += BWD_EFF * w.d * pairs[b]
    return tasks, flop, len(heads)


def cpu_baseline(names, workers):
    """Time the oracle (as it stands) on the host cores, before any GPU use.

    Every workload of ``names`` gets a bounded sample of whole (b, h)
    slices (all of them for the small workloads, one per worker for the
    long-context one) run by a fork pool of ``workers`` processes with one
    BLAS thread each; the headline workload is also timed on one worker
    (one slice).  Returns {name: dict}."""
    import multiprocessing as mp
    from entmax_amd.workloads import WORKLOADS, make_inputs
    for name in names:
        _CPU_INPUTS[name] = make_inputs(name)
    ctx = mp.get_context("fork")
    res = {}
    with ctx.Pool(workers) as pool:
        for name in names:
            w = WORKLOADS[name]
            n_heads = workers if w.L > 2048 else w.B * w.H
            tasks, flop, nh = _cpu_tasks(name, n_heads)
            t0 = time.perf_counter()
            pool.map(_cpu_task, tasks, chunksize=1)
            dt = time.perf_counter() - t0
            res[name] = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
                         "sample": f"{nh} whole (batch, head) slices of the {name} workload "
                                   f"({'forward+backward' if w.backward else 'forward'}, float64 numpy, "
                                   f"{workers} worker processes with one BLAS thread each), {dt:.1f} s wall"}
    if HEADLINE in names:
        tasks, flop, nh = _cpu_tasks(HEADLINE, 1)
        t0 = time.perf_counter()
        for t in tasks:
            _cpu_task(t)
        dt = time.perf_counter() - t0
        res[HEADLINE]["one_worker"] = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": 1,
                                       "sample": f"{nh} whole (batch, head) slice, forward+backward, {dt:.1f} s"}
    _CPU_INPUTS.clear()
    return res


def cpu_workers():
    """Worker processes for the CPU baseline: the cores this process may run
    on, at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
# GPU timing of the attention workloads
# ---------------------------------------------------------------------------

def time_workload(name, steps, warmup, copy_gbs):
    """Warm up, then time exactly ``steps`` steps of one workload; returns a
    result dict (ms per step, effective TFLOP/s, roofline of its longest call,
    zero fraction)."""
    import torch
    from entmax_amd import (bwd_workspace_bytes, entmax_attn_bwd_saved, entmax_attn_fwd, entmax_attn_fwd_save,
                            entmax_attn_probs, saved_bytes)
    from entmax_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    inp = make_inputs(name)
    dev = torch.device("cuda:0")
    km_cpu = inp["key_mask"]
    pairs = sum(allowed_pairs_per_head(w, km_cpu)) * w.H
    eff_flop = FWD_EFF * w.d * pairs + (BWD_EFF * w.d * pairs if w.backward else 0)

    # rotating buffer sets, > 512 MB in total
    esz = 4 if w.dtype == "f32" else 2
    n_el = w.B * w.H * w.L * w.d
    set_bytes = n_el * (3 * esz + 4) + w.B * w.H * w.L * 4
    ws_bytes = bwd_workspace_bytes(w.B, w.H, w.L, w.d) if w.backward else 0
    sv_bytes = saved_bytes(w.B, w.H, w.L, w.d) if w.backward else 0
    if w.backward:
        set_bytes += n_el * (esz + 12) + ws_bytes + sv_bytes
    nsets = max(2, min(64, math.ceil(2 * MALL_BYTES / set_bytes)))
    sets = []
    for _ in range(nsets):
        s = {x: inp[x].to(dev) for x in ("q", "k", "v")}
        s["key_mask"] = None if km_cpu is None else km_cpu.to(dev)
        s["out"] = torch.empty((w.B, w.H, w.L, w.d), dtype=torch.float32, device=dev)
        s["tau"] = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=dev)
        if w.backward:
            s["dout"] = inp["dout"].to(dev)
            s["grads"] = [torch.empty((w.B, w.H, w.L, w.d), dtype=torch.float32, device=dev) for _ in range(3)]
            s["ws"] = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
            s["saved"] = torch.empty((max(sv_bytes, 1),), dtype=torch.uint8, device=dev)
        sets.append(s)
    torch.cuda.synchronize()

    # With a backward the forward keeps each row's support for it (as a
    # training step keeps what its backward needs) and the backward reads it.
    def step(s, mid=None):
        if not w.backward:
            entmax_attn_fwd(s["q"], s["k"], s["v"], s["key_mask"], w.causal, w.window, out=s["out"],
                            tau_out=s["tau"])
            return
        entmax_attn_fwd_save(s["q"], s["k"], s["v"], s["key_mask"], w.causal, w.window, out=s["out"],
                             tau_out=s["tau"], saved=s["saved"])
        if mid is not None:
            mid.record()   # between the forward and the backward call, same stream
        entmax_attn_bwd_saved(s["q"], s["k"], s["v"], s["tau"], s["dout"], s["saved"], s["key_mask"], w.causal,
                              w.window, dq=s["grads"][0], dk=s["grads"][1], dv=s["grads"][2], workspace=s["ws"])

    for i in range(warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()

    # nonzeros of A (outside the timed region), for the algorithmic FLOPs and
    # the zero fraction
    s0 = sets[0]
    nnz = 0
    hb = max(1, (2 ** 31) // (w.L * w.L * 4))      # heads per probs call (<= 2 GiB)
    for h0 in range(0, w.H, hb):
        sl = slice(h0, min(w.H, h0 + hb))
        q_, k_ = s0["q"][:, sl].contiguous(), s0["k"][:, sl].contiguous()
        t_ = s0["tau"][:, sl].contiguous()
        pr = entmax_attn_probs(q_, k_, t_, s0["key_mask"], w.causal, w.window)
        nnz += int((pr > 0).sum().item())
        del pr
    torch.cuda.synchronize()

    # Timed region: the steps back to back on the launch stream, HIP events
    # only at its ends (and, with a backward, one per step boundary plus one
    # between the two calls: those kernels run for milliseconds).  Per-launch
    # events around microsecond kernels would add gaps to the steps.
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    if w.backward:
        bounds = [ev() for _ in range(steps + 1)]
        mids = [ev() for _ in range(steps)]
        torch.cuda.synchronize()
        bounds[0].record()
        for i in range(steps):
            step(sets[i % nsets], mids[i])
            bounds[i + 1].record()
        torch.cuda.synchronize()
        total_ms = bounds[0].elapsed_time(bounds[-1])
        fwd_each = [bounds[i].elapsed_time(mids[i]) for i in range(steps)]
        bwd_each = [mids[i].elapsed_time(bounds[i + 1]) for i in range(steps)]
        fwd_ms, bwd_ms = sum(fwd_each) / steps, sum(bwd_each) / steps
        fwd_med, bwd_med = statistics.median(fwd_each), statistics.median(bwd_each)
    else:
        t_start, t_end = ev(), ev()
        torch.cuda.synchronize()
        t_start.record()
        for i in range(steps):
            step(sets[i % nsets])
        t_end.record()
        torch.cuda.synchronize()
        total_ms = t_start.elapsed_time(t_end)
        fwd_ms = fwd_med = total_ms / steps   # the forward call is the whole step
        bwd_ms = bwd_med = 0.0
    ms_per_step = total_ms / steps
    del sets
    torch.cuda.empty_cache()

    res = {"workload": name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "dtype": w.dtype, "causal": w.causal,
           "window": w.window, "padding": w.padding, "backward": w.backward, "allowed_pairs": pairs,
           "nnz": nnz, "zero_fraction": 1.0 - nnz / pairs, "buffer_sets": nsets, "steps": steps,
           "warmup": warmup, "ms_per_step": ms_per_step,
           "effective_tflops": eff_flop / (ms_per_step * 1e-3) / 1e12}
    peak = MFMA_F32_PEAK_TFLOPS if w.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
    res["effective_frac_of_mfma_peak"] = res["effective_tflops"] / peak
    if BOUND[name] == "hbm":
        bytes_per_launch = algorithmic_bytes(w, km_cpu)
        achieved = bytes_per_launch / (fwd_ms * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "kernel": "fwd_short", "achieved": achieved, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                           "frac_of_measured_copy": None if copy_gbs is None else achieved / copy_gbs,
                           "traffic": measured_traffic(name), "bytes_per_launch": bytes_per_launch,
                           "launch_ms": fwd_ms}
    else:
        fwd_flop = 2.0 * w.d * pairs + 2.0 * w.d * nnz
        fwd_roof = {"bound": "mfma", "kernel": "fwd", "achieved": fwd_flop / (fwd_ms * 1e-3) / 1e12,
                    "peak": peak, "unit": "TFLOP/s", "flop_per_launch": fwd_flop, "launch_ms": fwd_ms,
                    "launch_ms_median": fwd_med, "traffic": measured_traffic(name)}
        fwd_roof["frac"] = fwd_roof["achieved"] / peak
        res["roofline"] = fwd_roof
        if w.backward:
            # the backward reads the forward's saved support: gathers of the
            # kept entries' rows, no score recomputed, no MFMA
            bwd_bytes = saved_bwd_bytes(w, nnz)
            bwd_roof = {"bound": "hbm", "kernel": "bwd", "achieved": bwd_bytes / (bwd_ms * 1e-3) / 1e9,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "bytes_per_launch": bwd_bytes, "launch_ms": bwd_ms,
                        "launch_ms_median": bwd_med, "traffic": measured_traffic(name, "bwd")}
            bwd_roof["frac"] = bwd_roof["achieved"] / HBM_PEAK_GBS
            bwd_roof["frac_of_measured_copy"] = None if copy_gbs is None else bwd_roof["achieved"] / copy_gbs
            res["fwd_ms"], res["bwd_ms"] = fwd_ms, bwd_ms
            res["fwd_effective_tflops"] = FWD_EFF * w.d * pairs / (fwd_ms * 1e-3) / 1e12
            res["bwd_effective_tflops"] = BWD_EFF * w.d * pairs / (bwd_ms * 1e-3) / 1e12
            res["bwd_roofline"] = bwd_roof
            if bwd_ms > fwd_ms:
                res["roofline"], res["fwd_roofline"] = bwd_roof, fwd_roof
    return res


def bench_attention(args, names):
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from entmax_amd import load_library
    load_library()
    copy_gbs = copy_bandwidth()
    results = {}
    for name in names:
        print(f"[bench] {name}", file=sys.stderr, flush=True)
        results[name] = time_workload(name, args.steps, args.warmup, copy_gbs)
    return results, copy_gbs


def main_attention(args):
    names = ORDER if args.workload == "all" else (args.workload,)
    head = HEADLINE if args.workload == "all" else args.workload
    # The CPU baseline runs first, before anything touches the GPU (the
    # worker pool is forked).
    cpu = None if args.no_cpu_baseline else cpu_baseline(names, args.cpu_workers or cpu_workers())
    results, copy_gbs = bench_attention(args, names)
    h = results[head]
    res = {
        "metric": METRIC,
        "value": h["effective_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h["dtype"],
        "data": "synthetic",
        "config": {k: h[k] for k in ("workload", "B", "H", "L", "d", "causal", "window", "padding", "backward",
                                     "allowed_pairs", "nnz", "zero_fraction", "buffer_sets")},
        "roofline": h["roofline"],
        "cpu_baseline": None if cpu is None else cpu[head],
        "flop_convention": {"effective_per_pair": {"fwd": f"{FWD_EFF} d", "bwd": f"{BWD_EFF} d"},
                            "algorithmic": {"fwd": "2 d pairs + 2 d nnz",
                                            "bwd": "bytes: Q, K, V, dO read, tau and the saved support read, "
                                                   "dQ, dK, dV written (no score recomputed)"}},
        "measured_copy_gbs": copy_gbs,
    }
    for k in ("fwd_ms", "bwd_ms", "fwd_effective_tflops", "bwd_effective_tflops", "fwd_roofline", "bwd_roofline"):
        if k in h:
            res[k] = h[k]
    if len(names) > 1:
        res["configs"] = {}
        for name in names:
            r = results[name]
            entry = {"ms_per_step": r["ms_per_step"], "effective_tflops": r["effective_tflops"],
                     "effective_frac_of_mfma_peak": r["effective_frac_of_mfma_peak"],
                     "roofline": {k: r["roofline"].get(k) for k in ("bound", "kernel", "achieved", "peak", "unit",
                                                                    "frac", "frac_of_measured_copy", "traffic")},
                     "zero_fraction": r["zero_fraction"], "shape": f"B{r['B']} H{r['H']} L{r['L']} d{r['d']} "
                                                                  f"{r['dtype']}",
                     "cpu_baseline": None if cpu is None else cpu.get(name)}
            for k in ("fwd_ms", "bwd_ms", "fwd_effective_tflops", "bwd_effective_tflops"):
                if k in r:
                    entry[k] = r[k]
            res["configs"][name] = entry
    print(json.dumps(res))


# ---------------------------------------------------------------------------
# Row-wise op and decode time (separate workloads, not part of the metric)
# ---------------------------------------------------------------------------

def bench_rows(args):
    """The row-wise op (forward + backward on a [R, L] score matrix), HBM-bound."""
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from entmax_amd.workloads import make_row_inputs
        from oracle import entmax15_exact
        inp = make_row_inputs("rows")
        s64 = inp["scores"].to(__import__("torch").float64).numpy()
        done, t0 = 0, time.perf_counter()
        with threadpool_limits(limits=1):
            while time.perf_counter() - t0 < args.cpu_budget:
                entmax15_exact(s64[done % s64.shape[0]:done % s64.shape[0] + 256])
                done += 256
        dt = time.perf_counter() - t0
        L = s64.shape[1]
        cpu = {"value": done * L * 6 / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} rows of the rows workload, forward only (float64 numpy, one thread), {dt:.1f} s"}
    import torch
    from entmax_amd import entmax15_rows, entmax15_rows_bwd
    from entmax_amd.workloads import make_row_inputs
    inp = make_row_inputs("rows")
    R, L = inp["spec"]["R"], inp["spec"]["L"]
    dev = torch.device("cuda:0")
    fwd_bytes = R * L * (2 + 4) + R * 4          # read bf16 scores, write fp32 p and tau
    bwd_bytes = R * L * 12                        # read p and dp, write ds
    nsets = max(2, math.ceil(2 * MALL_BYTES / (fwd_bytes + R * L * 8)))
    sets = [{"s": inp["scores"].to(dev), "dp": inp["dp"].to(dev),
             "p": torch.empty((R, L), device=dev), "tau": torch.empty((R,), device=dev),
             "ds": torch.empty((R, L), device=dev)} for _ in range(nsets)]
    torch.cuda.synchronize()

    def step(s, mid=None):
        entmax15_rows(s["s"], p=s["p"], tau=s["tau"])
        if mid is not None:
            mid.record()
        entmax15_rows_bwd(s["p"], s["dp"], ds=s["ds"])

    for i in range(args.warmup):
        step(sets[i % nsets])
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    bounds = [ev() for _ in range(args.steps + 1)]
    mids = [ev() for _ in range(args.steps)]
    torch.cuda.synchronize()
    bounds[0].record()
    for i in range(args.steps):
        step(sets[i % nsets], mids[i])
        bounds[i + 1].record()
    torch.cuda.synchronize()
    fwd_ms = sum(bounds[i].elapsed_time(mids[i]) for i in range(args.steps)) / args.steps
    bwd_ms = sum(mids[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)) / args.steps
    ms_per_step = bounds[0].elapsed_time(bounds[-1]) / args.steps
    fwd_gbs = fwd_bytes / (fwd_ms * 1e-3) / 1e9
    res = {
        "metric": "row-wise 1.5-entmax fwd+bwd: effective GB/s (HBM roofline)",
        "value": (fwd_bytes + bwd_bytes) / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "rows", "R": R, "L": L, "buffer_sets": nsets},
        "roofline": {"bound": "hbm", "kernel": "rows_fwd", "achieved": fwd_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": fwd_gbs / HBM_PEAK_GBS, "traffic": None,
                     "bytes_per_launch": fwd_bytes, "launch_ms": fwd_ms},
        "cpu_baseline": cpu,
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "bwd_gbs": bwd_bytes / (bwd_ms * 1e-3) / 1e9,
    }
    print(json.dumps(res))


def bench_decode(args):
    """Decode time: one new query per sequence against a key/value cache,
    HBM-bound (one launch for spans of at most 256 keys, else four)."""
    import torch
    from entmax_amd import decode_workspace_bytes, entmax_attn_decode
    from entmax_amd.workloads import make_decode_inputs
    inp = make_decode_inputs(args.workload)
    w = inp["spec"]
    B, H, Hkv, S, d, W = w["B"], w["H"], w["Hkv"], w["S"], w["d"], w["window"]
    span = min(W, S) if W > 0 else S
    esz = 2 if w["dtype"] == "bf16" else 4
    # q, the span's K and V rows, O and tau, each moved once
    alg_bytes = B * H * d * esz + 2 * B * Hkv * span * d * esz + B * H * (d + 1) * 4
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from oracle import attention_decode
        done, t0 = 0, time.perf_counter()
        with threadpool_limits(limits=1):
            while time.perf_counter() - t0 < args.cpu_budget:
                b = done % B
                attention_decode(inp["q"][b:b + 1], inp["k"][b:b + 1], inp["v"][b:b + 1],
                                 inp["seqlens"][b:b + 1].numpy(), W)
                done += 1
        dt = time.perf_counter() - t0
        cpu = {"value": done * alg_bytes / B / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} sequences of the {args.workload} workload (float64 numpy, one thread), {dt:.1f} s"}
    dev = torch.device("cuda:0")
    cache_bytes = 2 * B * Hkv * S * d * esz
    nsets = max(2, math.ceil(2 * MALL_BYTES / cache_bytes))
    ws_bytes = decode_workspace_bytes(B, H, Hkv, S, d, W)
    sets = [{"q": inp["q"].to(dev), "k": inp["k"].to(dev), "v": inp["v"].to(dev), "sl": inp["seqlens"].to(dev),
             "ws": torch.empty((ws_bytes,), dtype=torch.uint8, device=dev),
             "out": torch.empty((B, H, d), device=dev), "tau": torch.empty((B, H), device=dev)}
            for _ in range(nsets)]
    torch.cuda.synchronize()

    def step(s):
        entmax_attn_decode(s["q"], s["k"], s["v"], s["sl"], W, out=s["out"], tau=s["tau"], workspace=s["ws"])

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    # A decode step is a few microseconds of GPU work, less than one Python
    # call through the binding: the steps are captured in a HIP graph of R
    # consecutive steps (R divides the step count) and the graph is replayed.
    R = max(r for r in range(1, 21) if args.steps % r == 0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(R):
            step(sets[i % nsets])
    graph.replay()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    t0, t1 = ev(), ev()
    t0.record()
    for _ in range(args.steps // R):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "decode-time 1.5-entmax attention: effective GB/s (HBM roofline)",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "H": H, "H_kv": Hkv, "S": S, "d": d, "window": W,
                   "buffer_sets": nsets, "graph_steps": R},
        "roofline": {"bound": "hbm",
                     "kernel": "dec_short (one launch)" if span <= 256 else "decode (scores, tau, P V, reduce: four launches)",
                     "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None, "bytes_per_launch": alg_bytes, "launch_ms": ms},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "tiny", "encoder", "long", "decoder", "longctx", "rows", "decode", "decode_long"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=0, help="worker processes for the CPU baseline (0: auto)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time (rows and decode)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device copy (byte-counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): every (batch, head) is independent, "
              "so the path shards by heads with no communication; run it once per GPU.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.workload == "rows":
        bench_rows(args)
        return
    if args.workload in ("decode", "decode_long"):
        bench_decode(args)
        return
    main_attention(args)


if __name__ == "__main__":
    main()
