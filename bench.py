"""Throughput of msign by Newton-Schulz on one MI355X.

Default: the square 8192 x 8192 bf16 workload (iid N(0,1)), 5-step quintic NS
with bf16 products, one msign per step.  Prints ONE JSON line with
matrices/s, effective TFLOP/s ((20 alpha + 10) n^3 per msign) as a fraction
of the bf16 dense MFMA peak (timed without events), the roofline of the
dominant kernel (a second pass of the same steps with HIP events on the launch
stream around that kernel's launches), comparisons the pages quote (the
symmetric X X^T against full-tile and library products, NS with full-tile
products, Gram against standard NS at alpha = 4 and 8) and the fp64 CPU
oracle timed on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--case NAME]
                  [--no-cpu] [--all OUT.jsonl]

`--case` picks another workload (see CASES); `--all` runs every case and
writes one JSON line per case to OUT.jsonl (the default line is still
printed).  Inputs are synthetic (seeded, see synthetic/) and already resident
in HBM when the timed region starts.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "msign matrices/s and effective TFLOP/s (% bf16 MFMA peak), T=5 NS, 1 GPU"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # MI355X dense MFMA
HBM_GBS = 8000.0

# name -> (workload, method, compute dtype, restarts); "ns_init" is standard NS
# with the improved initial normalisation, "muon_ns" a whole Muon step
# (momentum, msign by NS, parameter update) with the workload as gradients.
# Workloads of several shape groups run as one grouped call per step.
CASES = {
    "c3_ns_bf16": ("c3_8192x8192_bf16", "ns", "bf16", ()),
    "c3_ns_init_bf16": ("c3_8192x8192_bf16", "ns_init", "bf16", ()),
    "c1_ns_f32": ("c1_128x256_f32", "ns", "f32", ()),
    "c1_ns_bf16": ("c1_128x256_f32", "ns", "bf16", ()),
    "c2_ns_bf16": ("c2_1024x4096_bf16", "ns", "bf16", ()),
    "c2_gram_f16": ("c2_1024x4096_bf16", "gram", "f16", (2,)),
    "c4_ns_bf16": ("c4_block_bf16", "ns", "bf16", ()),
    "c4_muon_ns_bf16": ("c4_block_bf16", "muon_ns", "bf16", ()),
    "c5_ns_bf16": ("c5_moe_f16", "ns", "bf16", ()),
    "c5_gram_f16": ("c5_moe_f16", "gram", "f16", (2,)),
}
DEFAULT_CASE = "c3_ns_bf16"


def dense_flops(n, m, steps=5):
    """(20 alpha + 10) n^3 at T = 5: X X^T, A^2 and B X as dense GEMMs."""
    return steps * (4.0 * m * n * n + 2.0 * n ** 3)


def algorithmic_flops(n, m, method, steps=5):
    """Flops the method executes per msign ("Gram Newton-Schulz" §2.4 and
    §3.4 counts): symmetric NS T (3 alpha + 1) n^3; Gram NS with one restart
    (14 + 6 alpha) n^3 at T = 5."""
    if method == "gram":
        return (14.0 * n + 6.0 * m) * n * n
    return steps * (3.0 * m + n) * n * n


def mfma_loop_peak(M, dtype, launches=5, iters=20000):
    """TFLOP/s of the MFMA-only probe kernel (operands in registers, every
    SIMD busy): the matrix rate the chip sustains, clock limits included."""
    import torch
    from msign_newton_schulz_amd import _binding as B
    out = torch.empty(B.PROBE_BLOCKS * B.PROBE_THREADS, dtype=torch.float32, device="cuda")
    M.mfma_probe(2000, dtype, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flops = sum(M.mfma_probe(iters, dtype, out=out) for _ in range(launches))
    e1.record()
    torch.cuda.synchronize()
    return flops / (e0.elapsed_time(e1) * 1e-3) / 1e12


def class_flops(n, m, steps=5):
    """Algorithmic flops of one launch of each kernel class on one matrix
    ("Gram Newton-Schulz" §2.4 counts): a triangle product counts half of the
    dense work, so X X^T is m n^2, an n x n product n^3 and B X (or Q X)
    2 m n^2.  The whole-iteration kernel of small matrices computes every
    tile of its T steps: T (4 m n^2 + 2 n^3)."""
    return {"xxt": float(m) * n * n, "square": float(n) ** 3, "rect": 2.0 * m * n * n,
            "small": steps * (4.0 * m * n * n + 2.0 * n ** 3)}


def elementwise_bytes(rows, cols, method, io_bytes, c_bytes):
    """Algorithmic HBM bytes of the class-0 (HBM-bound) passes of one msign on
    one matrix: the sum of squares reads the input.  A wide input already in
    the compute dtype with cols a multiple of 64 is then read by the first
    products themselves (no other pass).  Otherwise the normalise pass reads
    it again and writes the fp32 master (NS only) and the compute-dtype copy,
    padded to 64 (rows and columns).  The improved initial normalisation adds
    its combine pass (reads A and A A, writes B).  In a Muon step the msign
    input is the fp32 M and the sum-of-squares pass also reads G and writes
    the updated M; the parameter update happens in the last product's
    epilogue (not counted here)."""
    pad = lambda v: (v + 63) // 64 * 64
    n, m = min(rows, cols), max(rows, cols)
    elems, padded = rows * cols, pad(n) * pad(m)
    x_bytes = 4 if method == "muon_ns" else io_bytes
    if method in ("ns", "gram", "ns_init") and rows <= cols and cols % 64 == 0 and io_bytes == c_bytes:
        b = elems * x_bytes
    else:
        b = 2 * elems * x_bytes + padded * (c_bytes + (0 if method == "gram" else 4))
    if method == "ns_init":
        b += 3 * pad(n) * pad(n) * c_bytes
    if method == "muon_ns":
        b += elems * (io_bytes + 4)
    return float(b)


# Counter summary of the dominant kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes, scaled by the same counters on a plain copy of known size).  Its
# traffic figure is reported only while the kernel sources hash to the value
# recorded with it; after any change to them it is stale and `traffic` is null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_nt_rect_8192x8192_bf16_traffic.md")
KERNEL_SOURCES = ("common.hpp", "gemm_nt.hpp", "init_scale.hpp", "launch.hpp", "launch_impl.hpp", "normalize.hpp",
                  "small_ns.hpp",
                  "msign_api.hip", "products_dense.hip", "products_grouped.hip", "products_single.hip")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "msign_newton_schulz_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload, kclass):
    """Bytes per launch from the committed counter summary, or None if there
    is none for this workload and kernel class or the sources changed."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if (fields.get("workload") != workload or fields.get("kernel class") != kclass
            or fields.get("source sha256") != kernel_source_hash()):
        return None
    try:
        return float(fields["traffic bytes per launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--case", default=DEFAULT_CASE, choices=sorted(CASES))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--all", default=None, help="run every case, one JSON line each, into this file")
    ap.add_argument("--no-timing", action="store_true", help="no per-kernel event timing")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the comparisons the default case carries (unit bench, dense NS, Gram vs NS)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of msign, run 3 plain device copies of this many bytes "
                         "(calibrates the HBM traffic counters)")
    return ap.parse_args()


def copy_calibration(nbytes):
    """Three device-to-device copies of `nbytes` with torch's copy kernel; the
    FETCH_SIZE/WRITE_SIZE counters of these dispatches give the scale of the
    counters against a known byte count."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "copies": 3}), flush=True)


def load_inputs(workload, device):
    import synthetic as S
    wl = S.WORKLOADS[workload]
    xs = [S.group_batch(g, device=device) for g in wl.groups]
    return wl, xs


def cpu_baseline(wl, method, sample_seconds=30.0):
    """The fp64 oracle on a bounded sample of the workload: its first matrix
    of the largest group, running 2 of the 5 steps (or all of them when that
    is cheap), scaled to matrices/s over the workload's mix."""
    import numpy as np
    import oracle as O
    import synthetic as S
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    cores = min(16, os.cpu_count() or 1)
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    try:
        if threadpool_info:
            used = [p.get("num_threads") for p in threadpool_info() if p.get("user_api") == "blas"]
            cores = int(used[0]) if used else cores
        per_matrix = []
        descr = []
        for g in wl.groups:
            m = S.as_f64(S.group_matrix(g, 0))
            n_, m_ = min(m.shape), max(m.shape)
            work = dense_flops(n_, m_)
            steps_run = 5 if work < 2e11 else 2
            t0 = time.perf_counter()
            if method == "ns":
                O.ns_single(m, steps=steps_run)
            elif method == "muon_ns":
                O.muon_step(0.02 * m, m, np.zeros_like(m), 0.95, 0.02,
                            msign=lambda v: O.ns_single(v, steps=steps_run))
            elif method == "ns_init":
                O.ns_improved_init_single(m, steps=steps_run)
            else:
                O.gram_ns_single(m, steps=steps_run, restart_after=(2,) if steps_run > 2 else ())
            dt = time.perf_counter() - t0
            per_matrix.append((g.batch, dt * 5.0 / steps_run))
            descr.append(f"{g.rows}x{g.cols}: {steps_run} of 5 steps on matrix 0"
                         + ("" if steps_run == 5 else ", scaled x5/2"))
        total = sum(b * t for b, t in per_matrix)
        nmat = sum(b for b, _ in per_matrix)
        return {"value": nmat / total, "unit": "matrices/s", "cores": cores,
                "host_cpu_count": os.cpu_count(), "kind": "oracle",
                "sample": "fp64 NumPy oracle (" + method + "), " + "; ".join(descr)
                          + f"; batch mix {[b for b, _ in per_matrix]} weighted"}
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)


def run_case(name, steps, warmup, with_cpu, with_timing, with_extras=False):
    import torch
    import msign_newton_schulz_amd as M

    workload, method, cdt, restarts = CASES[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl, xs = load_inputs(workload, dev)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[cdt]
    outs = [torch.empty_like(x) for x in xs]
    grouped = len(xs) > 1
    if method == "muon_ns":
        gen = torch.Generator(device=dev).manual_seed(77)
        params = [(0.02 * torch.randn(x.shape, generator=gen, device=dev)).to(x.dtype) for x in xs]
        moms = [torch.zeros(x.shape, dtype=torch.float32, device=dev) for x in xs]
    wss = []
    if not grouped and method != "muon_ns":
        b, r, c = xs[0].shape
        nb = (M.ns_workspace_bytes(b, r, c, tdt) if method.startswith("ns")
              else M.gram_ns_workspace_bytes(b, r, c, tdt))
        wss.append(torch.empty(max(nb, 1), dtype=torch.uint8, device=dev))

    def one_step():
        # grouped calls size their workspace themselves (torch's caching
        # allocator hands back the same block every step)
        if method == "muon_ns":
            M.muon_step(params, xs, moms, lr=0.02, mu=0.95, method="ns", compute_dtype=tdt)
        elif grouped and method.startswith("ns"):
            M.msign_ns_grouped(xs, compute_dtype=tdt, outs=outs, improved_init=(method == "ns_init"))
        elif grouped:
            M.msign_gram_ns_grouped(xs, compute_dtype=tdt, restart_after=restarts, outs=outs)
        elif method.startswith("ns"):
            M.msign_ns(xs[0], compute_dtype=tdt, out=outs[0], workspace=wss[0],
                       improved_init=(method == "ns_init"))
        else:
            M.msign_gram_ns(xs[0], compute_dtype=tdt, restart_after=restarts, out=outs[0], workspace=wss[0])

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    # the timed region: K whole steps, no events
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    probe = dom = ktime = None
    events_ms = None
    if with_timing:
        # one more step with every class timed: the per-class breakdown and
        # the dominant product class
        M.kernel_timing(True)
        one_step()
        torch.cuda.synchronize()
        probe = M.read_kernel_timing()
        M.kernel_timing(False)
        # roofline pass: the same K steps again, the dominant class's
        # launches bracketed by HIP events on the launch stream
        dom = max(("xxt", "square", "rect", "small"), key=lambda k: probe[k][0])
        M.kernel_timing(True, classes=[dom])
        torch.cuda.synchronize()
        p0 = time.perf_counter()
        for _ in range(steps):
            one_step()
        torch.cuda.synchronize()
        events_ms = 1e3 * (time.perf_counter() - p0) / steps
        ktime = M.read_kernel_timing()
        M.kernel_timing(False)

    elapsed = t1 - t0
    nmat = sum(x.shape[0] for x in xs)
    eff = 0.0
    alg = 0.0
    cls_flops = {"xxt": 0.0, "square": 0.0, "rect": 0.0, "small": 0.0}
    shapes = []
    for x in xs:
        b, r, c = x.shape
        n_, m_ = min(r, c), max(r, c)
        eff += b * dense_flops(n_, m_)
        alg += b * algorithmic_flops(n_, m_, method)
        shapes.append([int(b), int(r), int(c)])
        for k, v in class_flops(n_, m_).items():
            cls_flops[k] += b * v
    ms = 1e3 * elapsed / steps
    eff_tflops = eff * steps / elapsed / 1e12
    rec = {
        "metric": METRIC, "value": nmat * steps / elapsed, "unit": "matrices/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cdt, "data": "synthetic",
        "config": {"workload": workload, "case": name,
                   "method": {"ns": "msign_ns", "ns_init": "msign_ns_ex(IMPROVED_INIT)", "gram": "msign_gram_ns",
                              "muon_ns": "muon_step(MUON_NS)"}[method]
                   + ("_grouped" if grouped and method != "muon_ns" else ""),
                   "shapes": shapes, "T": 5, "compute": cdt, "restart_after": list(restarts),
                   "parallelism": "single GPU"},
        "effective_tflops": eff_tflops,
        "effective_frac_of_peak": eff_tflops / PEAK_TFLOPS[cdt],
        "algorithmic_tflops": alg * steps / elapsed / 1e12,
    }
    if events_ms is not None:
        rec["ms_per_step_roofline_pass"] = events_ms
    if ktime is not None:
        per = {}
        for k in ("normalize", "xxt", "square", "rect", "small"):
            tot, cnt = probe[k]
            per[k] = {"total_ms": tot, "launches": cnt, "avg_us": 1e3 * tot / cnt if cnt else None}
        rec["kernels_one_step"] = per
        # the HBM-bound passes (normalise and the like): algorithmic bytes of
        # one step over their event-timed duration in the probe step
        tot, cnt = probe["normalize"]
        if cnt and tot > 0:
            nbytes = 0.0
            for x in xs:
                b, r, c = x.shape
                nbytes += b * elementwise_bytes(r, c, method, x.element_size(),
                                                {"bf16": 2, "f16": 2, "f32": 4}[cdt])
            rec["normalize_hbm"] = {"bound": "hbm", "achieved": nbytes / (tot * 1e-3) / 1e9,
                                    "peak": HBM_GBS, "unit": "GB/s",
                                    "frac": nbytes / (tot * 1e-3) / 1e9 / HBM_GBS,
                                    "bytes_per_step": nbytes, "launches": cnt}
        tot, cnt = ktime[dom]
        if cnt:
            # one launch of a class processes every group's whole batch (a
            # grouped launch when there are several groups)
            flops_per_launch = cls_flops[dom]
            avg_s = tot / cnt / 1e3
            ach = flops_per_launch / avg_s / 1e12
            rec["roofline"] = {"bound": "mfma", "kernel": f"gemm_nt_kernel ({dom})", "achieved": ach,
                               "timed": "HIP events around each launch, roofline pass of K steps",
                               "peak": PEAK_TFLOPS[cdt], "unit": "TFLOP/s",
                               "frac": ach / PEAK_TFLOPS[cdt],
                               "traffic": recorded_traffic(workload, dom),
                               "avg_launch_us": avg_s * 1e6,
                               "algorithmic_flops_per_launch": flops_per_launch}
            if cdt in ("bf16", "f16"):
                # beside the published peak: the MFMA-only loop on this GPU
                loop = mfma_loop_peak(M, tdt)
                rec["mfma_loop_peak"] = {"value": loop, "unit": "TFLOP/s", "dtype": cdt,
                                         "kernel": "mfma_probe_kernel (16x16x32, operands in registers)"}
                rec["roofline"]["frac_of_loop_peak"] = ach / loop
                rec["effective_frac_of_loop_peak"] = eff_tflops / loop
    if with_extras and name == DEFAULT_CASE:
        rec.update(extras(M, xs[0], outs[0], ms))
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline(wl, method)
    return rec


def time_calls(fn, reps, warmup=2):
    """Milliseconds per call of fn over `reps` back-to-back calls (no events;
    synchronised on both sides)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    return 1e3 * (time.perf_counter() - t0) / reps


def extras(M, x, out, ns_ms):
    """Comparisons the headline workload's line carries (a few seconds):
    - syrk_unit: X X^T at 8192^2 bf16 by the triangle kernel (upper tiles,
      mirrored), by the same kernel on every tile, and by torch.matmul
      (hipBLASLt) of x and x.T, as in the flash-muon excerpt on nil9.net
      (its symmetric operator at dimension 8192 takes about half the
      native time), also with x.T copied to row-major first;
    - dense_products_ns: the same NS with X X^T and c A A + b A on every
      tile, the end-to-end saving of the symmetric products (the excerpt:
      0.71x of native NS time);
    - gram_vs_ns: Gram NS (fp16 products, restart after step 2) against
      standard NS (bf16 products) at alpha = 4 (the 1024 x 4096 spiked
      workload) and alpha = 8 (the 8 x 1024 x 8192 MoE group), where
      "Gram Newton-Schulz" §5.2 expects Gram NS to win.
    Other hardware's figures are context, not targets."""
    import torch
    import synthetic as S
    res = {}
    x0 = x[0:1]
    c = torch.empty((1, x.shape[1], x.shape[1]), dtype=x.dtype, device=x.device)
    t_tri = time_calls(lambda: M.syrk_xxt(x0, out=c), 10)
    t_full = time_calls(lambda: M.syrk_xxt(x0, out=c, full_tiles=True), 10)
    # the library product as the excerpt names it, matmul(x, x.T) (2-D, the
    # transposed operand as a view), and with X^T copied first (row-major
    # operands); the library picks a kernel on its first calls, so these
    # get more warm-up calls
    xm, xt = x0[0], x0[0].transpose(0, 1).contiguous()
    cm = c[0]
    t_torch = time_calls(lambda: torch.matmul(xm, xm.t(), out=cm), 10, warmup=5)
    t_torch_nn = time_calls(lambda: torch.matmul(xm, xt, out=cm), 10, warmup=5)
    n, k = x.shape[1], x.shape[2]
    res["syrk_unit"] = {
        "shape": [int(n), int(k)], "dtype": "bf16",
        "triangle_us": 1e3 * t_tri, "full_tiles_us": 1e3 * t_full, "torch_matmul_us": 1e3 * t_torch,
        "torch_matmul_row_major_operands_us": 1e3 * t_torch_nn,
        "triangle_over_full_tiles": t_tri / t_full, "triangle_over_torch_matmul": t_tri / t_torch,
        "triangle_algorithmic_tflops": float(k) * n * n / (t_tri * 1e-3) / 1e12,
        "context": "flash-muon excerpt (nil9.net): about 0.5x of native matmul at dimension 8192, "
                   "hardware not stated"}
    ws = torch.empty(max(M.ns_workspace_bytes(*x.shape, torch.bfloat16), 1), dtype=torch.uint8,
                     device=x.device)
    t_dense = time_calls(lambda: M.msign_ns(x, compute_dtype=torch.bfloat16, out=out, workspace=ws,
                                            dense_products=True), 3, warmup=1)
    res["dense_products_ns"] = {
        "ms": t_dense, "symmetric_ms": ns_ms, "symmetric_over_dense": ns_ms / t_dense,
        "context": "flash-muon excerpt (nil9.net): 0.71x end-to-end NS time, hardware not stated"}
    cmp = {}
    for label, workload, gi, reps in (("alpha4_1024x4096", "c2_1024x4096_bf16", 0, 50),
                                      ("alpha8_8x1024x8192", "c5_moe_f16", 1, 10)):
        xg = S.group_batch(S.WORKLOADS[workload].groups[gi], device=x.device)
        yg = torch.empty_like(xg)
        b, r, cc = xg.shape
        wn = torch.empty(max(M.ns_workspace_bytes(b, r, cc, torch.bfloat16), 1), dtype=torch.uint8,
                         device=x.device)
        wg = torch.empty(max(M.gram_ns_workspace_bytes(b, r, cc, torch.float16), 1), dtype=torch.uint8,
                         device=x.device)
        t_ns = time_calls(lambda: M.msign_ns(xg, compute_dtype=torch.bfloat16, out=yg, workspace=wn), reps)
        t_gr = time_calls(lambda: M.msign_gram_ns(xg, compute_dtype=torch.float16, restart_after=(2,),
                                                  out=yg, workspace=wg), reps)
        cmp[label] = {"shape": [int(b), int(r), int(cc)], "ns_bf16_ms": t_ns, "gram_f16_restart2_ms": t_gr,
                      "gram_over_ns": t_gr / t_ns}
    cmp["context"] = ("Gram Newton-Schulz §5.2: Gram NS cuts NS time by 40-50% at the aspect ratios "
                      "of MLP and MoE weights (Kimi K2, hardware not stated)")
    res["gram_vs_ns"] = cmp
    return res


def main():
    args = parse()
    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(msign shards by batch across GPUs, each GPU running its share with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    if args.all:
        with open(args.all, "w") as f:
            for name in CASES:
                print(f"[bench] case {name}", file=sys.stderr, flush=True)
                steps = args.steps if not name.startswith("c4") else max(3, args.steps // 4)
                rec = run_case(name, steps, args.warmup, with_cpu=False, with_timing=not args.no_timing)
                f.write(json.dumps(rec) + "\n")
                f.flush()
                print(f"[bench] {name}: {rec['value']:.4g} matrices/s, "
                      f"{rec['effective_tflops']:.1f} effective TFLOP/s", file=sys.stderr, flush=True)
    rec = run_case(args.case, args.steps, args.warmup, with_cpu=not args.no_cpu,
                   with_timing=not args.no_timing, with_extras=not args.no_extras)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
