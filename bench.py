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
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed launches for this long before the warm-up steps, so that the "
                         "timed steps run at the GPU's loaded clock (0: none)")
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
        import subprocess
        out = subprocess.run(["lscpu"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                             text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if "cpu_model" not in info:
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


def gpu_sysfs_paths():
    """sysfs files of the GPU: the shader clock table (pp_dpm_sclk, the current clock marked with
    '*') and the socket power (hwmon power1_input, microwatts)."""
    import glob
    return (sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")),
            sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input")))


def parse_sclk(text):
    """Current shader clock in MHz from a pp_dpm_sclk table (the line marked '*'), or None."""
    import re
    for line in text.splitlines():
        if line.rstrip().endswith("*"):
            m = re.search(r"(\d+)\s*[Mm]hz", line)
            if m:
                return int(m.group(1))
    return None


class ClockSampler:
    """Samples the shader clock and the socket power from sysfs in a background thread, about
    every millisecond (best effort: the record says null where the files are not readable)."""

    def __init__(self):
        import threading
        self.clk_paths, self.pwr_paths = gpu_sysfs_paths()
        self.samples = []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _read(self, path):
        try:
            with open(path) as f:
                return f.read()
        except OSError:
            return None

    def _run(self):
        while not self._stop.is_set():
            now = time.perf_counter()
            clk = [parse_sclk(t) for t in map(self._read, self.clk_paths) if t]
            clk = [c for c in clk if c]
            pwr = []
            for t in map(self._read, self.pwr_paths):
                try:
                    pwr.append(int(t) / 1e6)
                except (TypeError, ValueError):
                    pass
            if clk or pwr:
                self.samples.append((now, max(clk) if clk else None, sum(pwr) if pwr else None))
            time.sleep(0.001)

    def __enter__(self):
        if self.clk_paths or self.pwr_paths:
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.clk_paths or self.pwr_paths:
            self._t.join()

    def summary(self, t0, t1):
        xs = [(c, p) for (t, c, p) in self.samples if t0 <= t <= t1]
        if not xs:
            return None
        out = {"samples": len(xs)}
        c = sorted(v for v, _ in xs if v is not None)
        if c:
            out.update(median_mhz=c[len(c) // 2], min_mhz=c[0], max_mhz=c[-1])
        p = sorted(v for _, v in xs if v is not None)
        if p:
            out.update(median_w=round(p[len(p) // 2], 1))
        return out


def run_timed(step, stream, args):
    """The timing protocol of every leg. Untimed launches for --settle-ms of wall time (the GPU
    leaves its idle clock state: with only a few warm-up launches the first ~25 ms of load run at
    a lower clock), then --warmup untimed steps, then exactly --steps steps timed with HIP events on
    the launch stream, bracketed by device synchronisation. Returns (ms per step, wall seconds of
    the timed region, record fields)."""
    import torch
    extra = {}
    with ClockSampler() as clk:
        t_settle = time.perf_counter()
        n_settle = 0
        if args.settle_ms > 0:
            while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
                for _ in range(8):
                    step()
                n_settle += 8
                torch.cuda.synchronize()
        extra["settle"] = {"ms": round((time.perf_counter() - t_settle) * 1e3, 1),
                           "launches": n_settle}
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
        t1 = time.perf_counter()
    extra["clock_during_timed_steps"] = clk.summary(t0, t1)
    extra["clock_during_settle"] = clk.summary(t_settle, t_settle + extra["settle"]["ms"] / 1e3)
    return e0.elapsed_time(e1) / args.steps, t1 - t0, extra


def oracle_pool(tasks, budget_s=15.0, ram_bytes_per_task=0):
    """Run the oracle tasks (callables) on a pool of one worker per available core, with BLAS held
    to one thread per worker, in batches of one task per worker, going round the list again while
    time is left, until the budget is spent (at least one batch). Returns (task runs done, seconds,
    workers)."""
    import concurrent.futures as cf
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    workers = len(os.sched_getaffinity(0))
    if ram_bytes_per_task:
        try:
            avail = os.sysconf("SC_AVPHYS_PAGES") * os.sysconf("SC_PAGE_SIZE")
            workers = max(1, min(workers, int(avail * 0.5 // ram_bytes_per_task)))
        except (OSError, ValueError):
            pass
    import contextlib
    limit = threadpool_limits(limits=1, user_api="blas") if threadpool_limits else \
        contextlib.nullcontext()
    done, t0 = 0, time.perf_counter()
    workers = max(1, min(workers, len(tasks)))
    with limit, cf.ThreadPoolExecutor(max_workers=workers) as ex:
        while True:
            batch = [tasks[(done + i) % len(tasks)] for i in range(workers)]
            list(ex.map(lambda f: f(), batch))
            done += len(batch)
            if time.perf_counter() - t0 >= budget_s:
                break
    return done, time.perf_counter() - t0, workers


def cpu_baseline(q, k, v, scale, causal, w, n_heads, budget_s=15.0):
    """Time the float64 oracle, as it stands, on a bounded sample of the workload: whole heads (or,
    for workloads checked on sampled rows, those rows of every head), one head per worker."""
    import numpy as np
    from oracle import attention_head
    from exact_tiled_attention_05_amd import workloads as W
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    group = H // w.get("H_kv", H)  # query heads per K/V head
    rows = None
    if w.get("sample_rows"):
        rows = W.sampled_rows(N, w["sample_rows"], w["seed"])
    heads = [(b, h) for b in range(B) for h in range(H)][:n_heads]

    def task(b, h):
        def run():
            qh = q[b, h].float().numpy().astype(np.float64)
            kh, vh = (x[b, h // group].float().numpy().astype(np.float64) for x in (k, v))
            attention_head(qh, kh, vh, scale, causal, rows)
        return run

    R = N if rows is None else len(rows)
    done, dt, workers = oracle_pool([task(b, h) for b, h in heads], budget_s,
                                    ram_bytes_per_task=3 * R * N * 8)
    # (done counts head passes: the pool goes round the heads again while the budget lasts)
    if rows is None:
        flops = W.metric_flops(1, done, N, d, causal)
        what = "%d passes over %d of %d heads, every row" % (done, len(heads), B * H)
    else:
        per_row = [4 * ((i + 1) if causal else N) * d for i in rows]
        flops = done * float(sum(per_row))
        what = ("%d passes over %d of %d heads, the %d sampled rows of each (FLOPs 4*(i+1)*d per "
                "causal row i)" % (done, len(heads), B * H, len(rows)))
    return dict({"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
                 "sample": "%s; numpy float64 with dense S and P, one head per worker, BLAS at one "
                           "thread per worker, %.1f s" % (what, dt)}, **host_info())


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

    ms, wall, timing = run_timed(step, stream, args)
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
    rec.update(timing)
    if not args.no_cpu:
        group = H // H_kv

        def task(b, h):
            def run():
                qh = q[b, h].float().numpy().astype(np.float64)
                kh, vh = (x[b, h // group].float().numpy().astype(np.float64) for x in (k, v))
                attention_head(qh, kh, vh, scale, causal, query_offset=Nkv - Nq)
            return run

        done, dt, workers = oracle_pool([task(b, h) for b in range(B) for h in range(H)],
                                        ram_bytes_per_task=3 * Nq * Nkv * 8)
        # each (b, h) reads its K/V head once: bytes of the heads done, at the oracle's rate
        rec["cpu_baseline"] = {"value": done * Nkv * d * 2 * 2 / dt / 1e9, "unit": "GB/s",
                               "cores": workers, "kind": "oracle",
                               "sample": "%d passes over the %d (batch, head) pairs, numpy "
                                         "float64, one pair per worker, BLAS at one thread per "
                                         "worker, %.1f s" % (done, B * H, dt)}
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

    ms, wall, timing = run_timed(step, stream, args)
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
                   "kernel": "fa_fwd_ext (%s)" % device_kernel(args.workload)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(args.workload)},
        "wall_s_timed_region": round(wall, 4),
        "kernel_ms": per_launch_ms(step, stream),
    }
    rec.update(timing)
    if not args.no_cpu:
        group = H // H_kv
        sl = W.alibi_slopes(H).tolist() if w.get("alibi") else None
        bcpu = W.workload_bias(args.workload) if w.get("bias_seed") else None

        def task(h):
            def run():
                qh = q[0, h].float().numpy().astype(np.float64)
                kh, vh = (x[0, h // group].float().numpy().astype(np.float64) for x in (k, v))
                bm = bcpu[0, h].float().numpy().astype(np.float64) if bcpu is not None else None
                attention_head(qh, kh, vh, scale, causal, window=win,
                               alibi_slope=None if sl is None else sl[h], bias=bm)
            return run

        done, dt, workers = oracle_pool([task(h) for h in range(H)],
                                        ram_bytes_per_task=4 * N * N * 8)
        cflops = W.metric_flops_masked(1, done, N, d, causal, win)
        rec["cpu_baseline"] = {"value": cflops / dt / 1e12, "unit": "TFLOP/s", "cores": workers,
                               "kind": "oracle",
                               "sample": "%d passes over the %d heads of batch 0 (of %d), every "
                                         "row (numpy float64, dense S and P), one head per worker, "
                                         "BLAS at one thread per worker, %.1f s"
                                         % (done, H, B * H, dt)}
        rec["cpu_baseline"].update(host_info())
    print(json.dumps(rec), flush=True)


def bench_backward(args, w):
    """Backward workloads: one step = one fa_bwd call (the dQ kernel, then the dK/dV kernel, then
    with query-head splits the kernel that adds the partial dK/dV sums), with
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

    ms, wall, timing = run_timed(step, stream, args)
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
                   "kernel": "fa_bwd (fa_bwd_dq_kernel + fa_bwd_dkdv_wide_kernel at d = 128, "
                             "fa_bwd_dkdv_kernel at d = 64; + fa_bwd_combine_kernel with "
                             "query-head splits)",
                   "workspace_bytes": need},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(args.workload)},
        "wall_s_timed_region": round(wall, 4),
        "kernel_ms": per_launch_ms(step, stream),
    }
    rec.update(timing)
    if not args.no_cpu:
        group = H // H_kv

        def task(h):
            def run():
                qh, doh = (x[0, h].float().numpy().astype(np.float64) for x in (q, do))
                kh, vh = (x[0, h // group].float().numpy().astype(np.float64) for x in (k, v))
                attention_backward_head(qh, kh, vh, doh, scale, causal)
            return run

        done, dt, workers = oracle_pool([task(h) for h in range(H)],
                                        ram_bytes_per_task=6 * N * N * 8)
        cflops = W.metric_flops_bwd(1, done, N, d, causal)
        rec["cpu_baseline"] = {"value": cflops / dt / 1e12, "unit": "TFLOP/s", "cores": workers,
                               "kind": "oracle",
                               "sample": "%d passes over the %d heads of batch 0 (of %d), every "
                                         "row (numpy float64, dense S, P, dP, dS), one head per "
                                         "worker, BLAS at one thread per worker, %.1f s"
                                         % (done, H, B * H, dt)}
        rec["cpu_baseline"].update(host_info())
    print(json.dumps(rec), flush=True)


# Sources that decide the code a workload runs: the C-ABI file (argument checks, launch shapes,
# split and head-split plans), the header, the shared device helpers, and the kernel family.
_FAMILY_SOURCES = {
    "fwd": ("fa_fwd_bf16.h",),
    "wide": ("fa_fwd_wide.h", "fa_wide.hip", "fa_tiles.h"),
    "ext": ("fa_fwd_ext.h", "fa_tiles.h", "fa_fwd_bf16.h"),
    "decode": ("fa_decode.h",),
    "bwd": ("fa_bwd.h", "fa_bwd_wide.h", "fa_bwd_wide.hip", "fa_tiles.h"),
}


def workload_family(workload):
    from exact_tiled_attention_05_amd import workloads as W
    w = W.WORKLOADS[workload]
    if "Nq" in w:
        return "decode"
    if w.get("backward"):
        return "bwd"
    # fa_api.hip: bf16 d = 128 with N >= 4096 runs the wide-row kernel, plain, with a causal
    # sliding window or with causal ALiBi (alone); every other variant (bias, other windows, other
    # ALiBi) runs the 4-wave kernel, and so do d = 256, the rest of causal d = 128 and grids of
    # more than 2^16 query rows; the remaining small grids run the 8-wave kernel
    long128 = w["dtype"] == "bf16" and w["d"] == 128 and w["N"] >= 4096
    if w.get("bias_seed"):
        return "ext"
    if w.get("alibi"):
        return "wide" if long128 and w["causal"][-1] and not w.get("window") else "ext"
    if w.get("window"):
        return "wide" if long128 and w["causal"][-1] and w["window"][0] >= 0 else "ext"
    if long128:
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
        print("bench.py: the library runs on one GPU only (no multi-GPU path); "
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

    ms, wall, timing = run_timed(step, stream, args)

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
    rec.update(timing)
    if not args.no_cpu:
        n_heads = args.cpu_heads or w["B"] * w["H"]
        rec["cpu_baseline"] = cpu_baseline(q, k, v, scale, causal, w, n_heads)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
