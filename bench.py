"""Throughput of the complex chunkwise SSD scan on one MI355X.

Default workload: the full-network scan load of a 28-layer Mamba-3-Lite
(each layer B=32, T=2048, H=16, N=D=64, chunk 64; layer l drawn with seed l),
all 28 layers resident in HBM and scanned back to back. One step is one pass
over the 28 layers. Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

The line also carries side figures: the single-layer workloads (B=1, B=8) and
the backward (ssd_chunk_backward, all its passes) on layer 0 of the network
load. `--backward-only` times just that backward leg (for profiling runs).
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
KERNEL_SOURCE = os.path.join(ROOT, "complex_chunkwise_ssd_amd", "csrc", "ssd_kernels.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_scan_kernel_network_b32_t2048.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def measured_traffic(launch_tokens_heads):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


# The four counter runs behind the traffic record (<dir> is any output directory;
# `bench.py --write-traffic-profile <dir>` then reads them).
TRAFFIC_COMMANDS = [
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/pmc_fetch -o scan -- python -u bench.py --steps 1 --warmup 0 --layers 2 --no-extra --no-cpu-baseline --no-backward",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/pmc_write -o scan -- python -u bench.py --steps 1 --warmup 0 --layers 2 --no-extra --no-cpu-baseline --no-backward",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/pmc_fetch_copy -o copy -- python -u bench.py --copy-calibration-mib 1024",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/pmc_write_copy -o copy -- python -u bench.py --copy-calibration-mib 1024",
]


def write_traffic_profile(root):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE of the scan kernel, each scaled by the
    same counter on a plain 1 GiB device copy, written next to the kernel trace
    summary (the source hash ties the figures to the kernel they were taken on)."""
    import csv
    import glob

    def counter(sub, name, kernel_part):
        vals = []
        for f in glob.glob(os.path.join(root, sub, "**", "*counter_collection.csv"), recursive=True):
            per = {}
            for r in csv.DictReader(open(f)):
                if kernel_part in r["Kernel_Name"] and r["Counter_Name"] == name:
                    per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
            vals += list(per.values())
        if not vals:
            raise SystemExit("no %s records for %s under %s" % (name, kernel_part, sub))
        return vals

    fetch = counter("pmc_fetch", "FETCH_SIZE", "scan_kernel<64, 0>")
    write = counter("pmc_write", "WRITE_SIZE", "scan_kernel<64, 0>")
    cf = max(counter("pmc_fetch_copy", "FETCH_SIZE", "copyBuffer"))
    cw = max(counter("pmc_write_copy", "WRITE_SIZE", "copyBuffer"))
    copied = 1 << 30
    fs, ws = copied / (cf * 1024), copied / (cw * 1024)
    f_kib, w_kib = sum(fetch) / len(fetch), sum(write) / len(write)
    rd, wr = f_kib * 1024 * fs, w_kib * 1024 * ws
    import complex_chunkwise_ssd_amd as ssd
    th = 32 * 2048 * 16
    rec = {
        "kernel": "ssd::scan_kernel<64, 0>",
        "workload": "one layer of the 28-layer network load: B=32, T=2048, H=16, N=D=64, chunk 64",
        "kernel_source_sha256_16": kernel_source_hash(),
        "fetch_size_kib_per_dispatch": f_kib,
        "write_size_kib_per_dispatch": w_kib,
        "copy_calibration": {"bytes_copied": copied, "fetch_size_kib": cf, "write_size_kib": cw,
                             "fetch_scale": fs, "write_scale": ws},
        "hbm_read_bytes_per_launch": rd,
        "hbm_write_bytes_per_launch": wr,
        "hbm_bytes_per_launch": rd + wr,
        "algorithmic_bytes_per_launch": th * ssd.algorithmic_bytes_per_token_head(64, 64, 2048),
        "commands": TRAFFIC_COMMANDS,
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return 0


def _short_kernel_name(name):
    """`ssd::gemm_kernel<false, false, true>(ssd::GemmParams)` -> the part before the
    argument list; torch's long template names are cut to their first 60 characters."""
    base = name.split("(")[0] if name.startswith(("void ssd::", "ssd::")) else name
    base = base.replace("void ", "", 1)
    return base if len(base) <= 80 else base[:60] + "..."


def trace_summary(root, skip_first=0, match="ssd::"):
    """Per-kernel durations from the rocprofv3 kernel traces (*kernel_trace.csv)
    under `root`: all calls, and the steady state with each kernel's first
    `skip_first` dispatches (the warm-up calls) left out. Prints a markdown
    table and returns the rows."""
    import csv
    import glob
    import statistics

    per = {}
    for f in sorted(glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            if match and match not in r["Kernel_Name"]:
                continue
            d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            per.setdefault(_short_kernel_name(r["Kernel_Name"]), []).append(
                (int(r["Dispatch_Id"]), d))
    rows = []
    print("| Kernel | Calls | Steady calls | Median ns | Mean ns | Min ns | Max ns | "
          "All-call mean ns |")
    print("|---|---|---|---|---|---|---|---|")
    for name, calls in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        calls.sort()
        ds = [d for _, d in calls]
        steady = ds[skip_first:] or ds
        row = {"kernel": name, "calls": len(ds), "steady_calls": len(steady),
               "median_ns": statistics.median(steady), "mean_ns": statistics.fmean(steady),
               "min_ns": min(steady), "max_ns": max(steady), "all_mean_ns": statistics.fmean(ds)}
        rows.append(row)
        print("| `%s` | %d | %d | %s | %s | %s | %s | %s |" % (
            name, row["calls"], row["steady_calls"], format(int(row["median_ns"]), ","),
            format(int(row["mean_ns"]), ","), format(row["min_ns"], ","),
            format(row["max_ns"], ","), format(int(row["all_mean_ns"]), ",")))
    return rows


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(layer0, rows_all=32, rows_one=2):
    """The oracle's plain recurrence timed on the host cores, on a bounded sample
    of layer 0 (all 16 heads, full T): a float (complex64) build at -O3
    -march=native, compiled here for this host, on every core the process may
    use (batch rows 0..rows_all-1, OpenMP over sequences) and on one thread
    (rows 0..rows_one-1); and the double-precision parity build as it is used
    by the tests, on every core. Inputs are on the host before the clock starts."""
    import tempfile

    import oracle
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count()
    omp = os.environ.get("OMP_NUM_THREADS", "")
    cores = min(avail, int(omp)) if omp.isdigit() and int(omp) > 0 else avail
    A = layer0.A.cpu()
    T = layer0.x.shape[1]

    def sample(rows):
        return (layer0.x[:rows].cpu(), A, layer0.B_t[:rows].cpu(), layer0.C_t[:rows].cpu(),
                layer0.dt[:rows].cpu())

    def timed(lib, rows, threads):
        args = sample(rows)
        # untimed first call on a few tokens: thread start-up and first-touch paging
        oracle.scan(*(a if a is A else a[:, :16] for a in args), threads=threads, lib=lib)
        t = time.perf_counter()
        oracle.scan(*args, threads=threads, lib=lib)
        return time.perf_counter() - t

    tmp = tempfile.mkdtemp(prefix="ssd_oracle_f32_")
    f32 = oracle.load(oracle.build_timing(os.path.join(tmp, "liboracle_f32.so")))
    H = A.shape[0]
    all_threads = min(cores, rows_all * H)
    el_all = timed(f32, rows_all, all_threads)
    el_one = timed(f32, rows_one, 1)
    el_dbl = timed(oracle.load(), rows_all, all_threads)
    return {"value": rows_all * T / el_all, "unit": "tokens*layers/s", "cores": all_threads,
            "kind": "oracle",
            "sample": "layer 0, batch rows 0-%d, all %d heads, T=%d (%d sequences, %.2f s wall); "
                      "float build (-O3 -march=native), OpenMP over sequences"
                      % (rows_all - 1, H, T, rows_all * H, el_all),
            "cpu_model": _cpu_model(),
            "build": "gcc -O3 -march=native -fno-fast-math -DORACLE_REAL=float (complex64)",
            "single_thread": {"value": rows_one * T / el_one, "unit": "tokens*layers/s",
                              "cores": 1,
                              "sample": "layer 0, batch rows 0-%d, all %d heads (%d sequences, "
                                        "%.2f s wall)" % (rows_one - 1, H, rows_one * H, el_one)},
            "double_parity_build": {"value": rows_all * T / el_dbl, "unit": "tokens*layers/s",
                                    "cores": all_threads,
                                    "sample": "as the headline sample (%.2f s wall); gcc -O2, "
                                              "double" % el_dbl}}


def proj_leg(ssd, torch, ssd_inputs, B, T, H, N, D, Q, dev, reps=20, dtype=None):
    """The scan read straight from in_proj output rows (real x, B and C as
    real/imaginary blocks; ssd_chunk_forward_proj, bfloat16 rows with
    dtype=torch.bfloat16) at the network layer shape, layer 0's seed; median
    of `reps` event-timed calls."""
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=0, device=dev, dtype=dtype)
    elem = proj.element_size()
    y = torch.empty((B, T, H, D), device=dev)
    f = torch.empty((B, H, N, D), dtype=torch.complex64, device=dev)
    n = ssd.workspace_bytes(B, T, H, N, D, Q)
    wsp = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    call = lambda: ssd.chunk_forward_proj(proj, A, H, N, D, chunk_size=Q, y=y, final_state=f,
                                          workspace=wsp)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    th = B * T * H
    fl = th * ssd.proj_algorithmic_flops_per_token_head(N, D, Q)
    tf = fl / (ms * 1e-3) / 1e12
    del proj, y, f, wsp
    return {"workload": "network layer in the in_proj layout, %s rows (B=%d, T=%d, H=%d, N=D=%d, "
                        "chunk %d)" % ("bfloat16" if elem == 2 else "float32", B, T, H, N, Q),
            "median_ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP32_MFMA_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / PEAK_FP32_MFMA_TFLOPS,
                         "algorithmic_flops": fl,
                         "algorithmic_bytes": th * ssd.proj_algorithmic_bytes_per_token_head(
                             N, D, T, elem)}}


def mix_leg(ssd, torch, ssd_inputs, B, T, H, D, dev, reps=20):
    """The MIMO head mixer after the scan (ssd_head_mix: z = y W^T with a dense
    (H*D, H*D) W) and its gradients (ssd_head_mix_backward: grad_y = grad_z W,
    grad_W = grad_z^T y) at the network layer shape; median of `reps` calls
    each, bracketed by HIP events on the stream the library launches on. Each
    product is 2 M F^2 flops for ~500 flops per byte at F = 1024, so the bound
    is the fp32 MFMA peak."""
    y, W, gz = ssd_inputs.mix_case((B, T, H, D), seed=0, device=dev)
    F = H * D
    M = B * T
    z = torch.empty_like(y)
    gy = torch.empty_like(y)
    gW = torch.empty((F, F), device=dev)
    ws = torch.empty(max(ssd.head_mix_workspace_bytes(M, H, D), 1), dtype=torch.uint8,
                     device=dev)
    out = {"workload": "network layer y (B=%d, T=%d, H=%d, D=%d), dense W (%d, %d)"
                       % (B, T, H, D, F, F)}
    one = ssd.mix_algorithmic_flops(M, H, D)
    for name, call, flops, nbytes in (
            ("forward", lambda: ssd.head_mix(y, W, z=z), one,
             ssd.mix_algorithmic_bytes(M, H, D)),
            ("backward", lambda: ssd.head_mix_backward(y, W, gz, grad_y=gy, grad_W=gW,
                                                       workspace=ws), 2 * one,
             ssd.mix_algorithmic_bytes(M, H, D, backward=True))):
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            ev.append((a, b))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
        tf = flops / (ms * 1e-3) / 1e12
        out[name] = {"median_ms": ms, "tokens_per_s": M / (ms * 1e-3),
                     "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP32_MFMA_TFLOPS,
                                  "unit": "TFLOP/s", "frac": tf / PEAK_FP32_MFMA_TFLOPS,
                                  "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
                                  "achieved_hbm_GBs_algorithmic": nbytes / (ms * 1e-3) / 1e9}}
    del y, W, gz, z, gy, gW, ws
    return out


def sweep_leg(ssd, torch, ssd_inputs, dev, reps=10):
    """The long-context chunk-size sweep: B=4, T=8192, H=16, N=D=64, dt ~ N(0.5, 1),
    one input set for chunk 32, 64, 128 and 256; median of `reps` event-timed
    ssd_chunk_forward calls per chunk size. A chunk above 64 tokens is evaluated
    as 64-token sub-chunks (the same sums re-associated), so the roofline fraction
    is taken against the algorithmic count of the block size actually evaluated."""
    w = ssd_inputs.WORKLOADS["sweep_b4_t8192"]
    B, T, H, N, D = w["batch"], w["T"], w["H"], w["N"], w["D"]
    g = ssd_inputs.layer_case(B, T, H, N, D, seed=w["seed"], dt_mean=w["dt_mean"], device=dev)
    y = torch.empty((B, T, H, D), device=dev)
    f = torch.empty((B, H, N, D), dtype=torch.complex64, device=dev)
    out = {"workload": "B=%d, T=%d, H=%d, N=D=%d, dt ~ N(%.1f, 1), one input set" % (
        B, T, H, N, w["dt_mean"])}
    th = B * T * H
    for i, q in enumerate(w["chunks"]):
        n = ssd.workspace_bytes(B, T, H, N, D, q)
        wsp = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        call = lambda: ssd.chunk_forward(g.x, g.A, g.B_t, g.C_t, g.dt, chunk_size=q, y=y,
                                         final_state=f, workspace=wsp)
        # untimed calls; before the first chunk size for about a second, so that the
        # clock has settled also when the sweep runs alone (--sweep-only)
        t_end = time.time() + (1.0 if i == 0 else 0.0)
        for k in range(1 << 30):
            call()
            if k >= 2 and time.time() >= t_end:
                break
            if k % 64 == 63:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            ev.append((a, b))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
        qe = ssd.block_rows(q)
        fe = th * ssd.algorithmic_flops_per_token_head(N, D, qe)
        by = th * ssd.algorithmic_bytes_per_token_head(N, D, T)
        out["chunk_%d" % q] = {
            "median_ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "token_heads_per_s": th / (ms * 1e-3), "evaluated_block_rows": qe,
            "roofline_frac_mfma": fe / (ms * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS,
            "achieved_hbm_GBs_algorithmic": by / (ms * 1e-3) / 1e9}
        del wsp
    del g, y, f
    return out


def backward_proj_leg(ssd, torch, ssd_inputs, B, T, H, N, D, dev, reps=10, dtype=None):
    """ssd_chunk_backward_proj (gradients as in_proj gradient rows; bfloat16 rows
    and gradient rows with dtype=torch.bfloat16) at the network layer shape;
    median of `reps` event-timed calls."""
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=0, device=dev, dtype=dtype)
    gy, gf = ssd_inputs.upstream_grads(B, T, H, N, D, seed=0, device=dev)
    ws = torch.empty(max(ssd.backward_workspace_bytes(B, T, H, N, D, 64), 1), dtype=torch.uint8,
                     device=dev)
    rows = torch.zeros_like(proj)
    call = lambda: ssd.chunk_backward_proj(proj, A, H, N, D, gy, gf, chunk_size=64, grad_proj=rows,
                                           workspace=ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    del proj, gy, gf, ws, rows
    qe = ssd.backward_block_rows(64)
    fl = B * T * H * ssd.proj_backward_algorithmic_flops_per_token_head(N, D, qe)
    achieved = fl / (ms * 1e-3) / 1e12
    return {"workload": "network layer backward from %s in_proj rows (B=%d, T=%d, H=%d, "
                        "N=D=%d, chunk 64)" % ("bfloat16" if dtype == torch.bfloat16 else
                                              "float32", B, T, H, N),
            "median_ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP32_MFMA_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_MFMA_TFLOPS,
                         "scope": "whole call at the real-x algorithmic count",
                         "algorithmic_flops": fl, "evaluated_chunk": qe}}


def backward_leg(ssd, torch, g, reps=10, warmup=3):
    """ssd_chunk_backward on one network layer (B=32, T=2048, H=16, N=D=64,
    chunk 64) with seeded upstream gradients; median of `reps` calls, each
    bracketed by HIP events on the stream the library launches on."""
    import ssd_inputs
    B, T, H, D = g.x.shape
    N = g.B_t.shape[-1]
    Q = 64
    gy, gf = ssd_inputs.upstream_grads(B, T, H, N, D, seed=0, device=g.x.device)
    ws = torch.empty(max(ssd.backward_workspace_bytes(B, T, H, N, D, Q), 1), dtype=torch.uint8,
                     device=g.x.device)
    out = ssd.chunk_backward(g.x, g.A, g.B_t, g.C_t, g.dt, gy, gf, chunk_size=Q, workspace=ws)
    call = lambda: ssd.chunk_backward(g.x, g.A, g.B_t, g.C_t, g.dt, gy, gf, chunk_size=Q, out=out,
                                      workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    th = B * T * H
    qb = ssd.backward_block_rows(Q)
    fl = th * ssd.backward_algorithmic_flops_per_token_head(N, D, qb)
    by = th * ssd.backward_algorithmic_bytes_per_token_head(N, D, T)
    tf = fl / (ms * 1e-3) / 1e12
    del ws, out, gy, gf
    return {"workload": "network layer 0 backward (B=%d, T=%d, H=%d, N=D=%d, chunk %d)"
                        % (B, T, H, N, Q),
            "median_ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "token_heads_per_s": th / (ms * 1e-3),
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP32_MFMA_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / PEAK_FP32_MFMA_TFLOPS,
                         "scope": "whole call: state pass, adjoint pass, chunk pass, gA sum",
                         "algorithmic_flops": fl, "algorithmic_bytes": by,
                         "evaluated_chunk": qb}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="network_28x_b32_t2048")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the single-layer side figures")
    ap.add_argument("--layers", type=int, default=None,
                    help="override the layer count (counter runs; the headline uses all layers)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward side figure")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward on layer 0 of the workload and print it")
    ap.add_argument("--sweep-only", action="store_true",
                    help="time only the T=8192 chunk-size sweep and exit")
    ap.add_argument("--mix-only", action="store_true",
                    help="time only the MIMO head mixer (forward and gradients) and exit")
    ap.add_argument("--write-traffic-profile", metavar="DIR", default=None,
                    help="read the four rocprofv3 FETCH_SIZE / WRITE_SIZE runs (scan and a "
                         "1 GiB copy) under DIR and write the committed traffic summary")
    ap.add_argument("--trace-summary", metavar="DIR", default=None,
                    help="print per-kernel steady-state durations from the rocprofv3 kernel "
                         "traces under DIR and exit")
    ap.add_argument("--skip-first", type=int, default=0,
                    help="with --trace-summary: warm-up dispatches of each kernel to leave out")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this size (HBM counter calibration)")
    args = ap.parse_args()
    if args.write_traffic_profile:
        return write_traffic_profile(args.write_traffic_profile)
    if args.trace_summary:
        trace_summary(args.trace_summary, args.skip_first)
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (the (batch, head) "
              "sequences are independent, so they would shard over GPUs with no communication)",
              file=sys.stderr)
        return 2

    import torch

    import complex_chunkwise_ssd_amd as ssd
    import ssd_inputs

    dev = torch.device("cuda:0")
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "copies": 3}))
        return 0
    wl = dict(ssd_inputs.WORKLOADS[args.workload])
    B, T, H, N, D = wl["batch"], wl["T"], wl["H"], wl["N"], wl["D"]
    if args.sweep_only:
        print(json.dumps({"chunk_sweep": sweep_leg(ssd, torch, ssd_inputs, dev,
                                                   reps=max(args.steps, 1))}), flush=True)
        return 0
    if args.mix_only:
        print(json.dumps({"head_mix": mix_leg(ssd, torch, ssd_inputs, B, T, H, D, dev,
                                              reps=max(args.steps, 1))}), flush=True)
        return 0
    if args.backward_only:
        g = ssd_inputs.layer_case(B, T, H, N, D, seed=0 if wl["seed"] is None else wl["seed"],
                                  dt_mean=wl["dt_mean"], device=dev)
        print(json.dumps({"backward": backward_leg(ssd, torch, g, reps=max(args.steps, 1),
                                                   warmup=args.warmup)}), flush=True)
        return 0
    Q = wl["chunks"][0]
    L = wl.get("layers", 1) if args.layers is None else args.layers
    log("bench: workload %s (%d layer(s) of B=%d T=%d H=%d N=%d D=%d Q=%d)" % (args.workload, L, B, T,
                                                                                 H, N, D, Q))
    layers, ys, fss = [], [], []
    for l in range(L):
        seed = l if wl["seed"] is None else wl["seed"]
        layers.append(ssd_inputs.layer_case(B, T, H, N, D, seed=seed, dt_mean=wl["dt_mean"],
                                            device=dev))
        ys.append(torch.empty((B, T, H, D), dtype=torch.float32, device=dev))
        fss.append(torch.empty((B, H, N, D), dtype=torch.complex64, device=dev))
    wsn = ssd.workspace_bytes(B, T, H, N, D, Q)
    ws = torch.empty(max(wsn, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log("bench: inputs resident (%.1f GB)" % (torch.cuda.memory_allocated() / 1e9))

    def step(ev=None):
        for l, g in enumerate(layers):
            if ev is not None:
                ev[l][0].record()
            ssd.chunk_forward(g.x, g.A, g.B_t, g.C_t, g.dt, chunk_size=Q, y=ys[l], final_state=fss[l],
                              workspace=ws)
            if ev is not None:
                ev[l][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("bench: warmup done")

    per_launch = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(L)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(args.steps):
        step(per_launch[k])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    launch_ms = [a.elapsed_time(b) for row in per_launch for a, b in row]
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    log("bench: %d steps in %.1f ms (wall %.2f s), %.3f ms per layer call" % (args.steps, total_ms,
                                                                            wall, avg_launch_ms))

    th_per_launch = B * T * H
    flops_launch = th_per_launch * ssd.algorithmic_flops_per_token_head(N, D, Q)
    bytes_launch = th_per_launch * ssd.algorithmic_bytes_per_token_head(N, D, T)
    achieved = flops_launch / (avg_launch_ms * 1e-3) / 1e12
    tokens_layers = B * T * L
    value = tokens_layers / (ms_per_step * 1e-3)
    traffic = measured_traffic(th_per_launch)
    out = {
        "metric": "complex-SSD scan tokens/s at T=2048,H=16,N=D=64,Q=64 + % of roofline",
        "value": value,
        "unit": "tokens*layers/s" if L > 1 else "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; shapes and value ranges of the Mamba-3-Lite pages)",
        "config": {"workload": args.workload, "layers": L, "batch": B, "seq_len": T, "heads": H,
                   "state_N": N, "head_dim_D": D, "chunk_size": Q},
        "token_heads_per_s": value * H,
        "tokens_per_s_network": B * T / (ms_per_step * 1e-3),
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_FP32_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_MFMA_TFLOPS,
            "traffic": traffic,
            "kernel": "scan_kernel<64, 0> (complex layout; one launch per layer)",
            "avg_launch_ms": avg_launch_ms,
            "algorithmic_flops_per_launch": flops_launch,
            "algorithmic_bytes_per_launch": bytes_launch,
            "achieved_hbm_GBs_algorithmic": bytes_launch / (avg_launch_ms * 1e-3) / 1e9,
            "kernel_source_sha256_16": kernel_source_hash(),
        },
    }

    if not args.no_extra:
        extra = {}
        for name in ("layer_b1_t2048", "layer_b8_t2048"):
            w = ssd_inputs.WORKLOADS[name]
            g = ssd_inputs.layer_case(w["batch"], w["T"], w["H"], w["N"], w["D"], seed=w["seed"],
                                      device=dev)
            q = w["chunks"][0]
            y = torch.empty((w["batch"], w["T"], w["H"], w["D"]), device=dev)
            f = torch.empty((w["batch"], w["H"], w["N"], w["D"]), dtype=torch.complex64, device=dev)
            n = ssd.workspace_bytes(w["batch"], w["T"], w["H"], w["N"], w["D"], q)
            wsp = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
            call = lambda: ssd.chunk_forward(g.x, g.A, g.B_t, g.C_t, g.dt, chunk_size=q, y=y,
                                             final_state=f, workspace=wsp)
            for _ in range(5):
                call()
            torch.cuda.synchronize()
            times = []
            for _ in range(50):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                call()
                b.record()
                times.append((a, b))
            torch.cuda.synchronize()
            ms = sorted(a.elapsed_time(b) for a, b in times)[len(times) // 2]
            th = w["batch"] * w["T"] * w["H"]
            fl = th * ssd.algorithmic_flops_per_token_head(w["N"], w["D"], q)
            by = th * ssd.algorithmic_bytes_per_token_head(w["N"], w["D"], w["T"])
            extra[name] = {"median_ms": ms, "tokens_per_s": w["batch"] * w["T"] / (ms * 1e-3),
                           "token_heads_per_s": th / (ms * 1e-3),
                           "roofline_frac_mfma": fl / (ms * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS,
                           "achieved_hbm_GBs_algorithmic": by / (ms * 1e-3) / 1e9}
            del g, y, f, wsp
        out["single_layer"] = extra
        out["proj_layer"] = proj_leg(ssd, torch, ssd_inputs, B, T, H, N, D, Q, dev)
        out["proj_layer_bf16"] = proj_leg(ssd, torch, ssd_inputs, B, T, H, N, D, Q, dev,
                                          dtype=torch.bfloat16)
        out["head_mix"] = mix_leg(ssd, torch, ssd_inputs, B, T, H, D, dev)
        out["chunk_sweep"] = sweep_leg(ssd, torch, ssd_inputs, dev)
    if not args.no_backward:
        log("bench: timing the backward on layer 0")
        out["backward"] = backward_leg(ssd, torch, layers[0])
        if not args.no_extra:
            out["backward_proj"] = backward_proj_leg(ssd, torch, ssd_inputs, B, T, H, N, D, dev)
            out["backward_proj_bf16"] = backward_proj_leg(ssd, torch, ssd_inputs, B, T, H, N, D,
                                                          dev, dtype=torch.bfloat16)

    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(layers[0])
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
