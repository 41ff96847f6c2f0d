#!/usr/bin/env python3
"""Throughput of the exact tiled attention forward pass on one MI355X.

One step = one fa_fwd call over the whole workload (grid, Q load, K/V streaming, both MFMA
contractions, online softmax, epilogue), with Q, K, V already resident in HBM. The default
workload is the Llama-3-8B layer shape: B=1, H=32, N=8192, d=128, bf16, causal.

Prints one JSON line:
  value      = metric FLOPs (4*B*H*N^2*d, halved when causal) / mean step time, in TFLOP/s
  roofline   = the kernel's achieved TFLOP/s against the dense bf16 MFMA peak, timed with HIP
               events on the stream the kernel is launched on
  cpu_baseline = the CPU float64 oracle timed on this host on a bounded sample of the workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_F32_TFLOPS = 157.3    # MI355X fp32 vector


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b_n8k_causal")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="max heads in the cpu_baseline sample (0 = all, capped at ~15 s)")
    ap.add_argument("--print-digest", action="store_true",
                    help="print the kernel source digest that recorded counters are keyed to")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="BYTES",
                    help="instead of attention, run --steps plain device copies of BYTES bytes "
                         "(reference kernel for scaling the HBM byte counters)")
    return ap.parse_args()


def host_info():
    """Cores available, CPU model and BLAS library of this host (for the cpu_baseline record)."""
    info = {"cores_available": len(os.sched_getaffinity(0))}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = "%s %s" % (blas[0].get("internal_api"), blas[0].get("version"))
    except Exception:  # pragma: no cover
        pass
    return info


def per_launch_ms(step, stream, n=20):
    """Median and minimum of n individually event-timed launches, run after the timed region
    (each one alone on the idle GPU, so they include no queueing behind other launches)."""
    import torch
    ts = []
    for _ in range(n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    return {"median": round(ts[len(ts) // 2], 5), "min": round(ts[0], 5), "launches": n}


def copy_calibration(nbytes, steps):
    """A plain device-to-device copy of known size: reads and writes nbytes per launch."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": steps}), flush=True)


def cpu_baseline(q, k, v, scale, causal, w, n_heads, budget_s=15.0):
    """Time the float64 oracle, as it stands, on whole heads (all their rows), in order, until
    n_heads heads are done or budget_s seconds have passed (at least one head)."""
    import numpy as np
    from oracle import attention_head
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    heads = [(b, h) for b in range(w["B"]) for h in range(w["H"])][:n_heads]
    dt = 0.0
    done = 0
    group = w["H"] // w.get("H_kv", w["H"])  # query heads per K/V head
    for b, h in heads:
        qh = q[b, h].float().numpy().astype(np.float64)
        kh, vh = (x[b, h // group].float().numpy().astype(np.float64) for x in (k, v))
        t0 = time.perf_counter()
        attention_head(qh, kh, vh, scale, causal)
        dt += time.perf_counter() - t0
        done += 1
        if dt >= budget_s:
            break
    from exact_tiled_attention_05_amd.workloads import metric_flops
    flops = metric_flops(1, done, w["N"], w["d"], causal)
    return dict({"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                 "sample": "%d of %d heads, every row (numpy float64, dense S and P), %.1f s"
                           % (done, w["B"] * w["H"], dt)}, **host_info())


def bench_decode(args, w):
    """Split-KV decoding workloads: one step = one fa_fwd_splitkv call (both kernels), with the
    workspace allocated once beforehand. Reported as K/V bytes read per second (the quantity the
    step is bound by) against the HBM peak."""
    import numpy as np
    import torch
    import exact_tiled_attention_05_amd as fa
    from exact_tiled_attention_05_amd import workloads as W
    from oracle import attention_head

    causal = w["causal"][-1]
    q, k, v, scale = W.workload_inputs(args.workload)
    B, H, H_kv, Nq, Nkv, d = w["B"], w["H"], w["H_kv"], w["Nq"], w["N"], w["d"]
    layout = w.get("layout", "bhnd")
    lay = fa.FA_LAYOUT_BHND if layout == "bhnd" else fa.FA_LAYOUT_BNHD
    dev = torch.device("cuda:0")
    qd, kd, vd = (W.to_layout(x, layout).to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    need = fa.fa_splitkv_workspace_bytes(B, H, H_kv, Nq, Nkv, d, int(causal), 0)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    argv = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H_kv,
            Nq, Nkv, d, scale, int(causal), lay, 0, ws.data_ptr(), need, stream.cuda_stream)

    def step():
        rc = fa.fa_fwd_splitkv(*argv)
        if rc != fa.FA_OK:
            raise fa.FAError(rc, "fa_fwd_splitkv")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    kv_bytes = 2 * B * H_kv * Nkv * d * 2
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    # algorithmic bytes of the step: K, V and Q read once, O and LSE written once (the split
    # partials' round trip through the workspace is the method's overhead, not counted)
    alg = kv_bytes + 2 * (B * H * Nq * d * 2) + B * H * Nq * 4
    alg_gbs = alg / (ms * 1e-3) / 1e9
    rec = {
        "metric": "attention decode K/V bytes read per second (2*B*H_kv*N_kv*d*2 bytes per step)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q, K, V)",
        "config": {"workload": args.workload, "B": B, "H": H, "H_kv": H_kv, "N_q": Nq, "N_kv": Nkv,
                   "d": d, "causal": causal, "layout": layout,
                   "kernel": "fa_fwd_splitkv (fa_decode_partial_kernel + fa_decode_combine_kernel)",
                   "workspace_bytes": need},
        "roofline": {"bound": "hbm", "achieved": round(alg_gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(alg_gbs / 8000.0, 4), "traffic": recorded_traffic(args.workload),
                     "algorithmic_bytes": alg},
        "wall_s_timed_region": round(wall, 4),
        "kernel_ms": per_launch_ms(step, stream),
    }
    if not args.no_cpu:
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()
                           if i.get("user_api") == "blas"] or [1])
        except Exception:  # pragma: no cover
            threads = 1
        group = H // H_kv
        dt, done = 0.0, 0
        for b in range(B):
            for h in range(H):
                qh = q[b, h].float().numpy().astype(np.float64)
                kh, vh = (x[b, h // group].float().numpy().astype(np.float64) for x in (k, v))
                t1 = time.perf_counter()
                attention_head(qh, kh, vh, scale, causal, query_offset=Nkv - Nq)
                dt += time.perf_counter() - t1
                done += 1
                if dt >= 15.0:
                    break
            if dt >= 15.0:
                break
        # each (b, h) reads its K/V head once: bytes of the heads done, at the oracle's rate
        rec["cpu_baseline"] = {"value": done * Nkv * d * 2 * 2 / dt / 1e9, "unit": "GB/s",
                               "cores": threads, "kind": "oracle",
                               "sample": "%d of %d (batch, head) pairs, numpy float64, %.1f s"
                                         % (done, B * H, dt)}
        rec["cpu_baseline"].update(host_info())
    print(json.dumps(rec), flush=True)


def bench_variant(args, w):
    """Score-variant workloads (sliding window, ALiBi, additive bias): one step = one fa_fwd_ext
    call. Reported in TFLOP/s of the visible (query, key) pairs, 4*d FLOPs each."""
    import numpy as np
    import torch
    import exact_tiled_attention_05_amd as fa
    from exact_tiled_attention_05_amd import workloads as W
    from oracle import attention_head

    causal = w["causal"][-1]
    q, k, v, scale = W.workload_inputs(args.workload)
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    H_kv = w.get("H_kv", H)
    layout = w.get("layout", "bhnd")
    lay = fa.FA_LAYOUT_BHND if layout == "bhnd" else fa.FA_LAYOUT_BNHD
    window = w.get("window", (-1, -1))
    dev = torch.device("cuda:0")
    qd, kd, vd = (W.to_layout(x, layout).to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    slopes = W.alibi_slopes(H).to(dev) if w.get("alibi") else None
    bias = W.workload_bias(args.workload).to(dev) if w.get("bias_seed") else None
    stream = torch.cuda.current_stream(dev)
    argv = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H_kv,
            N, d, scale, int(causal), lay, window[0], window[1],
            slopes.data_ptr() if slopes is not None else None,
            bias.data_ptr() if bias is not None else None, 0,
            bias.stride(1) if bias is not None else 0, bias.stride(2) if bias is not None else 0,
            stream.cuda_stream)

    def step():
        rc = fa.fa_fwd_ext(*argv)
        if rc != fa.FA_OK:
            raise fa.FAError(rc, "fa_fwd_ext")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    win = None if tuple(window) == (-1, -1) else tuple(window)
    flops = W.metric_flops_masked(B, H, N, d, causal, win)
    tflops = flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": "attention fwd TFLOP/s (4*d per visible query-key pair)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q, K, V%s)" % (", bias" if bias is not None else ""),
        "config": {"workload": args.workload, "B": B, "H": H, "H_kv": H_kv, "N": N, "d": d,
                   "causal": causal, "layout": layout, "window": list(window),
                   "alibi": bool(w.get("alibi")), "bias": bias is not None,
                   "kernel": "fa_fwd_ext (fa_fwd_ext_kernel)"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(args.workload)},
        "wall_s_timed_region": round(wall, 4),
        "kernel_ms": per_launch_ms(step, stream),
    }
    if not args.no_cpu:
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()
                           if i.get("user_api") == "blas"] or [1])
        except Exception:  # pragma: no cover
            threads = 1
        group = H // H_kv
        sl = W.alibi_slopes(H).tolist() if w.get("alibi") else None
        bcpu = W.workload_bias(args.workload) if w.get("bias_seed") else None
        dt, done = 0.0, 0
        for h in range(H):
            qh = q[0, h].float().numpy().astype(np.float64)
            kh, vh = (x[0, h // group].float().numpy().astype(np.float64) for x in (k, v))
            bm = bcpu[0, h].float().numpy().astype(np.float64) if bcpu is not None else None
            t1 = time.perf_counter()
            attention_head(qh, kh, vh, scale, causal, window=win,
                           alibi_slope=None if sl is None else sl[h], bias=bm)
            dt += time.perf_counter() - t1
            done += 1
            if dt >= 15.0:
                break
        cflops = W.metric_flops_masked(1, done, N, d, causal, win)
        rec["cpu_baseline"] = {"value": cflops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
                               "kind": "oracle",
                               "sample": "%d of %d heads of batch 0, every row (numpy float64, "
                                         "dense S and P), %.1f s" % (done, B * H, dt)}
        rec["cpu_baseline"].update(host_info())
    print(json.dumps(rec), flush=True)


def bench_backward(args, w):
    """Backward workloads: one step = one fa_bwd call (the dQ kernel, then the dK/dV kernel), with
    O and the logsumexp from one forward call and the workspace allocated before the timed
    region. Reported in TFLOP/s of the five gradient products (10*B*H*N^2*d, halved if causal)."""
    import numpy as np
    import torch
    import exact_tiled_attention_05_amd as fa
    from exact_tiled_attention_05_amd import workloads as W
    from oracle import attention_backward_head

    causal = w["causal"][-1]
    q, k, v, scale = W.workload_inputs(args.workload)
    do = W.workload_grad(args.workload)
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    H_kv = w.get("H_kv", H)
    layout = w.get("layout", "bhnd")
    lay = fa.FA_LAYOUT_BHND if layout == "bhnd" else fa.FA_LAYOUT_BNHD
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (W.to_layout(x, layout).to(dev) for x in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, scale=scale, causal=causal, layout=layout)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    need = fa.fa_bwd_workspace_bytes(B, H, H_kv, N, d)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    argv = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), dod.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, H_kv, N, d, scale,
            int(causal), lay, ws.data_ptr(), need, stream.cuda_stream)

    def step():
        rc = fa.fa_bwd(*argv)
        if rc != fa.FA_OK:
            raise fa.FAError(rc, "fa_bwd")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    flops = W.metric_flops_bwd(B, H, N, d, causal)
    tflops = flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": "attention bwd TFLOP/s (10*B*H*N^2*d, 1/2 if causal)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q, K, V, dO)",
        "config": {"workload": args.workload, "B": B, "H": H, "H_kv": H_kv, "N": N, "d": d,
                   "causal": causal, "layout": layout,
                   "kernel": "fa_bwd (fa_bwd_dq_kernel + fa_bwd_dkdv_kernel)",
                   "workspace_bytes": need},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(args.workload)},
        "wall_s_timed_region": round(wall, 4),
        "kernel_ms": per_launch_ms(step, stream),
    }
    if not args.no_cpu:
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()
                           if i.get("user_api") == "blas"] or [1])
        except Exception:  # pragma: no cover
            threads = 1
        group = H // H_kv
        dt, done = 0.0, 0
        for h in range(H):
            qh, doh = (x[0, h].float().numpy().astype(np.float64) for x in (q, do))
            kh, vh = (x[0, h // group].float().numpy().astype(np.float64) for x in (k, v))
            t1 = time.perf_counter()
            attention_backward_head(qh, kh, vh, doh, scale, causal)
            dt += time.perf_counter() - t1
            done += 1
            if dt >= 15.0:
                break
        cflops = W.metric_flops_bwd(1, done, N, d, causal)
        rec["cpu_baseline"] = {"value": cflops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
                               "kind": "oracle",
                               "sample": "%d of %d heads of batch 0, every row (numpy float64, "
                                         "dense S, P, dP, dS), %.1f s" % (done, B * H, dt)}
        rec["cpu_baseline"].update(host_info())
    print(json.dumps(rec), flush=True)


# Sources that decide the code a workload runs: the C-ABI file (argument checks, launch shapes,
# split and head-split plans), the header, the shared device helpers, and the kernel family.
_FAMILY_SOURCES = {
    "fwd": ("fa_fwd_bf16.h",),
    "wide": ("fa_fwd_wide.h", "fa_wide.hip", "fa_tiles.h"),
    "ext": ("fa_fwd_ext.h", "fa_tiles.h", "fa_fwd_bf16.h"),
    "decode": ("fa_decode.h",),
    "bwd": ("fa_bwd.h", "fa_tiles.h"),
}


def workload_family(workload):
    from exact_tiled_attention_05_amd import workloads as W
    w = W.WORKLOADS[workload]
    if "Nq" in w:
        return "decode"
    if w.get("backward"):
        return "bwd"
    # fa_api.hip: every variant runs the 4-wave kernel; plain bf16 d = 128 with N >= 4096 the
    # wide-row kernel; d = 256, the rest of causal d = 128 and grids of more than 2^16 query rows
    # the 4-wave kernel; the remaining small grids the 8-wave kernel
    if w.get("window") or w.get("alibi") or w.get("bias_seed"):
        return "ext"
    if w["dtype"] == "bf16" and w["d"] == 128 and w["N"] >= 4096:
        return "wide"
    if (w["d"] == 256 or (w["dtype"] == "bf16" and ((w["d"] == 128 and w["causal"][-1])
                                                    or w["B"] * w["H"] * w["N"] > (1 << 16)))):
        return "ext"
    return "fwd"


def _code_only(text):
    """C++ source without comments and with whitespace runs collapsed (a comment edit leaves the
    digest, and the counters keyed to it, unchanged)."""
    import re
    token = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|/\*.*?\*/|//[^\n]*', re.S)
    text = token.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
    return " ".join(text.split())


def device_kernel(workload):
    """Name of the device kernel the forward entry point runs for this workload (fa_api.hip picks
    it by shape)."""
    from exact_tiled_attention_05_amd import workloads as W
    w = W.WORKLOADS[workload]
    if w["dtype"] != "bf16":
        return "fa_fwd_f32_kernel"
    if workload_family(workload) == "wide":
        return "fa_fwd_wide_kernel, the wide-row kernel"
    if workload_family(workload) == "ext":
        return "fa_fwd_ext_kernel, the 4-wave kernel"
    return "fa_fwd_bf16_kernel, the 8-wave kernel"


def kernel_source_digest(workload):
    """sha256 over the build flags and the code (comments stripped) of the HIP sources of the
    kernels this workload runs (so a change to another kernel family leaves its recorded counters
    valid)."""
    import hashlib
    from exact_tiled_attention_05_amd import build as B
    hsh = hashlib.sha256()
    files = [os.path.join(B.CSRC, n) for n in
             ("fa_api.hip", "fa_device.h") + _FAMILY_SOURCES[workload_family(workload)]]
    files.append(os.path.join(B.INCLUDE, "fa.h"))
    for path in files:
        with open(path, encoding="utf-8") as f:
            hsh.update(os.path.basename(path).encode() + b"\0" + _code_only(f.read()).encode())
    hsh.update(" ".join(B.HIP_FLAGS).encode())
    return hsh.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per launch recorded with rocprofv3 counters for this workload, if they were
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != kernel_source_digest(workload):
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on exactly one GPU (no multi-GPU path); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.print_digest:
        print(kernel_source_digest(args.workload))
        return
    if args.copy_calib:
        copy_calibration(args.copy_calib, args.steps)
        return

    import torch
    import exact_tiled_attention_05_amd as fa
    from exact_tiled_attention_05_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    if "Nq" in w:
        return bench_decode(args, w)
    if w.get("backward"):
        return bench_backward(args, w)
    if w.get("window") or w.get("alibi") or w.get("bias_seed"):
        return bench_variant(args, w)
    causal = w["causal"][-1]
    q, k, v, scale = W.workload_inputs(args.workload)
    layout = w.get("layout", "bhnd")
    H_kv = w.get("H_kv", w["H"])
    dev = torch.device("cuda:0")
    qd, kd, vd = (W.to_layout(x, layout).to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w["B"], w["H"], w["N"]), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr())
    if layout == "bhnd" and H_kv == w["H"]:
        fn = fa.fa_fwd if w["dtype"] == "bf16" else fa.fa_fwd_f32
        argv = ptrs + (w["B"], w["H"], w["N"], w["d"], scale, int(causal), stream.cuda_stream)
    else:
        fn = fa.fa_fwd_gqa if w["dtype"] == "bf16" else fa.fa_fwd_gqa_f32
        lay = fa.FA_LAYOUT_BHND if layout == "bhnd" else fa.FA_LAYOUT_BNHD
        argv = ptrs + (w["B"], w["H"], H_kv, w["N"], w["d"], scale, int(causal), lay,
                       stream.cuda_stream)

    def step():
        rc = fn(*argv)
        if rc != fa.FA_OK:
            raise fa.FAError(rc, fn.__name__)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Events are recorded on the stream the kernels are launched on.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps

    flops = W.metric_flops(w["B"], w["H"], w["N"], w["d"], causal)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w["dtype"] == "bf16" else PEAK_F32_TFLOPS

    rec = {
        "metric": "attention fwd TFLOP/s (4*B*H*N^2*d, 1/2 if causal)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded N(0,1) Q, K, V)",
        "config": {"workload": args.workload, "B": w["B"], "H": w["H"], "H_kv": H_kv,
                   "N": w["N"], "d": w["d"], "causal": causal, "layout": layout,
                   "kernel": "%s (%s)" % (fn.__name__, device_kernel(args.workload))},
        "roofline": {"bound": "mfma" if w["dtype"] == "bf16" else "alu",
                     "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": recorded_traffic(args.workload)},
        "wall_s_timed_region": round(wall, 4),
        "kernel_ms": per_launch_ms(step, stream),
    }
    if not args.no_cpu:
        n_heads = args.cpu_heads or w["B"] * w["H"]
        rec["cpu_baseline"] = cpu_baseline(q, k, v, scale, causal, w, n_heads)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
