"""Throughput of 1.5-entmax attention on one MI355X, against its roofline.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole path over one batch of synthetic input:
the forward (scores, masks, row max, tau by bisection, P, O = P V) for the
forward workloads, forward + backward for ``longctx``.  Inputs are already
resident in HBM when the timed region starts; the timed steps rotate over
enough copies of the input/output buffers (> 256 MB in total) that no step is
served from the 256 MB Infinity Cache.

Prints ONE JSON line.  ``value`` is effective TFLOP/s: 4 d FLOPs per allowed
(query, key) pair for the forward (two products of d multiply-adds; zeros of
A count as done), plus 6 d per pair for the backward.  ``roofline`` reports
the dominant kernel: its algorithmic bytes (HBM-bound workloads) or
algorithmic MFMA FLOPs (MFMA-bound ones) per launch over its average launch
time, measured with HIP events on the launch stream over the timed region
(forward-only steps: the region over the step count; forward + backward:
events at the step boundaries and between the two launches).
``cpu_baseline`` times the float64 oracle on a bounded sample of the same
workload on the host cores.
"""

import argparse
import json
import math
import os
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

BOUND = {"tiny": "hbm", "encoder": "hbm", "long": "mfma", "decoder": "hbm", "longctx": "mfma"}


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
    """HBM bytes per launch of the workload's forward (or backward) kernel,
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


def cpu_baseline(name, budget_s=12.0):
    """Time the oracle (as it stands) on a bounded sample of the workload."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from entmax_amd.workloads import WORKLOADS, make_inputs
    from oracle import attention_backward, attention_forward

    w = WORKLOADS[name]
    inp = make_inputs(name)
    pairs = allowed_pairs_per_head(w, inp["key_mask"])
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    flop_per_pair = 4 * w.d + (6 * w.d if w.backward else 0)
    done_flop = 0.0
    n_heads = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            b, h = heads[n_heads % len(heads)]
            attention_forward(inp["q"], inp["k"], inp["v"], inp["key_mask"], w.causal, w.window, heads=[(b, h)])
            if w.backward:
                attention_backward(inp["q"], inp["k"], inp["v"], inp["dout"], inp["key_mask"], w.causal,
                                   w.window, heads=[(b, h)])
            done_flop += flop_per_pair * pairs[b]
            n_heads += 1
            if time.perf_counter() - t0 > budget_s and n_heads >= 1:
                break
    dt = time.perf_counter() - t0
    return {
        "value": done_flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{n_heads} (batch, head) slices of the {name} workload "
                  f"({'forward+backward' if w.backward else 'forward'}, float64 numpy, one thread), "
                  f"{dt:.1f} s",
    }


def bench_rows(args):
    """The row-wise op (forward + backward on a [R, L] score matrix), HBM-bound."""
    cpu = None
    if not args.no_cpu_baseline:
        import numpy as np
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
    ev = lambda: torch.cuda.Event(enable_timing=True)
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
        import numpy as np
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
    ev = lambda: torch.cuda.Event(enable_timing=True)
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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="encoder",
                    choices=["tiny", "encoder", "long", "decoder", "longctx", "rows", "decode", "decode_long"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device copy (byte-counter calibration) and exit")
    args = ap.parse_args()

    if args.copy_probe:
        copy_probe()
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): every (batch, head) is independent, "
              "so the path shards by heads with no communication; run it once per GPU.", file=sys.stderr)
        sys.exit(2)

    if args.workload == "rows":
        bench_rows(args)
        return
    if args.workload in ("decode", "decode_long"):
        bench_decode(args)
        return

    # The CPU baseline runs first, before anything touches the GPU.
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.workload, args.cpu_budget)

    import torch
    from entmax_amd import entmax_attn_bwd, entmax_attn_fwd
    from entmax_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    inp = make_inputs(args.workload)
    dev = torch.device("cuda:0")
    km_cpu = inp["key_mask"]
    pairs = sum(allowed_pairs_per_head(w, km_cpu)) * w.H
    fwd_flop = 4.0 * w.d * pairs
    bwd_flop = 6.0 * w.d * pairs if w.backward else 0.0

    # rotating buffer sets, > 256 MB in total
    esz = 4 if w.dtype == "f32" else 2
    n_el = w.B * w.H * w.L * w.d
    set_bytes = n_el * (3 * esz + 4) + w.B * w.H * w.L * 4
    if w.backward:
        set_bytes += n_el * (esz + 12)
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
        sets.append(s)
    torch.cuda.synchronize()

    def step(s, mid=None):
        entmax_attn_fwd(s["q"], s["k"], s["v"], s["key_mask"], w.causal, w.window, out=s["out"], tau_out=s["tau"])
        if w.backward:
            if mid is not None:
                mid.record()   # between the forward and the backward launch, same stream
            entmax_attn_bwd(s["q"], s["k"], s["v"], s["tau"], s["dout"], s["key_mask"], w.causal, w.window,
                            dq=s["grads"][0], dk=s["grads"][1], dv=s["grads"][2])

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()

    # nonzeros of A (outside the timed region), for the algorithmic FLOPs
    nnz = None
    if BOUND[args.workload] == "mfma":
        from entmax_amd import entmax_attn_probs
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
    # between the two launches: those kernels run for milliseconds).  Per-launch
    # events around microsecond kernels would add gaps to the steps.
    ev = lambda: torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if w.backward:
        bounds = [ev() for _ in range(args.steps + 1)]
        mids = [ev() for _ in range(args.steps)]
        bounds[0].record()
        for i in range(args.steps):
            step(sets[i % nsets], mids[i])
            bounds[i + 1].record()
        torch.cuda.synchronize()
        total_ms = bounds[0].elapsed_time(bounds[-1])
        fwd_ms = sum(bounds[i].elapsed_time(mids[i]) for i in range(args.steps)) / args.steps
        bwd_ms = sum(mids[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)) / args.steps
    else:
        t_start, t_end = ev(), ev()
        t_start.record()
        for i in range(args.steps):
            step(sets[i % nsets])
        t_end.record()
        torch.cuda.synchronize()
        total_ms = t_start.elapsed_time(t_end)
        fwd_ms = total_ms / args.steps   # the forward launch is the whole step
        bwd_ms = 0.0
    ms_per_step = total_ms / args.steps

    value = (fwd_flop + bwd_flop) / (ms_per_step * 1e-3) / 1e12

    # roofline of the dominant kernel
    bound = BOUND[args.workload]
    if bound == "hbm":
        bytes_per_launch = algorithmic_bytes(w, km_cpu)
        achieved = bytes_per_launch / (fwd_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "fwd", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(w.name),
                "bytes_per_launch": bytes_per_launch, "launch_ms": fwd_ms}
    else:
        peak = MFMA_F32_PEAK_TFLOPS if w.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
        if w.backward and bwd_ms > fwd_ms:
            # S recomputed for every allowed pair; dP, dQ, dK, dV on the support
            kname, kms = "bwd", bwd_ms
            flop = 2.0 * w.d * pairs + 8.0 * w.d * nnz
        else:
            # Q K^T for every allowed pair; P V on the support
            kname, kms = "fwd", fwd_ms
            flop = 2.0 * w.d * pairs + 2.0 * w.d * nnz
        achieved = flop / (kms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": kname, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": measured_traffic(w.name, kname),
                "flop_per_launch": flop, "launch_ms": kms}

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "causal": w.causal,
                   "window": w.window, "padding": w.padding, "backward": w.backward,
                   "allowed_pairs": pairs, "buffer_sets": nsets,
                   "zero_fraction": None if nnz is None else 1.0 - nnz / pairs},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if w.backward:
        res["fwd_ms"] = fwd_ms
        res["bwd_ms"] = bwd_ms
    print(json.dumps(res))


if __name__ == "__main__":
    main()
