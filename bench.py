#!/usr/bin/env python3
"""Benchmark of the exact residue GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload wide]

One step is one whole product C = A @ B on device-resident inputs: the residue
split of both operands (kernel 1), the 29 per-prime INT8 MFMA products with
the mod-q epilogue (kernel 2) and the reconstruction (kernel 3: the centered
CRT by rounded quotient, its sum over primes on the matrix cores).  Garner
reconstruction, which gives the same output, is timed after the step for
its share.  The
default workload is the widest of the five: A[2048,4096] @ B[4096,2048] with
2-limb entries uniform in [-2^100, 2^100), 29 primes, 4-limb output.

Prints one JSON line: the exact-GEMM rate 2*M*N*K / t_step, the roofline of
the dominant kernel (the per-prime INT8 products against the dense INT8 MFMA
peak), per-stage times, and the CPU oracle timed on a bounded sample of the
same workload on the host cores (a baseline, not a target).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "exact int GEMM ops/s (2MNK/s) + % of MI355X dense INT8 MFMA peak"
PEAK_INT8_TOPS = 5000.0        # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E, 8 TB/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wide",
                    choices=["tiny", "square", "enclosure", "dixon", "wide", "enclosure_fp64", "solve", "sliced"])
    ap.add_argument("--n", type=int, default=1024, help="system size of --workload solve")
    ap.add_argument("--rhs", type=int, default=1, help="right-hand sides of --workload solve")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the CPU oracle sample")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the shader clock with amd-smi (profiler runs)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only the int8 matrix-core ceiling (random and zero operand bytes)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 1 GiB device copy (calibrates HBM byte counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "gemm_wide_hbm_traffic.txt")
KERNEL_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exact_integer_gemm_amd",
                             "csrc", "rns_gemm.hip")


def measured_traffic(workload):
    """HBM bytes per GEMM launch from the committed counter summary, or None.

    The summary records the SHA-256 of the kernel source it was taken with;
    once the source has changed the figure no longer describes the kernel.
    """
    import hashlib
    if workload != "wide" or not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line:
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256") != src:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def gemm_kernel_name(tile_config, n, M, N):
    """The product kernels of the tiling the library chose (the layout's tile_config)."""
    import torch
    if tile_config == 2:
        return "gemm_kernel<128,32,64,4,1> (skinny tiles)"
    if tile_config == 1:
        return "gemm_kernel<64,64,64,2,2> (small tiles)"
    tiles = n * ((M + 255) // 256) * ((N + 255) // 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if tiles > cus and cus % 8 == 0:
        return ("gemm_ps_kernel<4> (persistent, one workgroup per CU) + gemm_tail4_kernel<8> "
                "when tiles past the last whole round are split over K")
    return "gemm_pp_kernel<4> (one 256x256 tile per workgroup)"


def spread(samples_ms):
    """Median, min and max of per-step stage times, in microseconds."""
    a = np.asarray(samples_ms, dtype=np.float64) * 1e3
    return {"median": float(np.median(a)), "min": float(a.min()), "max": float(a.max())}


def output_digest(workload, C):
    """SHA-256 of the output bytes next to the oracle's digest of the same workload."""
    import hashlib
    got = hashlib.sha256(np.ascontiguousarray(C.cpu().numpy()).tobytes()).hexdigest()
    ref = None
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests", "golden", "workload_digests.json")
    if os.path.exists(path):
        entry = json.load(open(path)).get(workload)
        if entry and entry.get("out_limbs") == C.shape[-1]:
            ref = entry.get("C_sha256")
    return {"output_sha256": got, "oracle_sha256": ref,
            "matches_oracle": (got == ref) if ref is not None else None}


def gfx_clock_during(run, seconds=1.5):
    """Median shader clock (MHz, mean over the XCDs) and socket power (W) that
    amd-smi reports while run() is called back to back for about `seconds`;
    (None, None) where amd-smi is not available."""
    import subprocess
    import threading
    import torch
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-c", "-p", "--json"], capture_output=True,
                                   text=True, timeout=10)
                g = json.loads(r.stdout)["gpu_data"][0]
                clk = [v["clk"]["value"] for k, v in g["clock"].items() if k.startswith("gfx_")]
                pw = g["power"]["socket_power"]["value"]
                samples.append((float(np.mean(clk)), float(pw)))
            except Exception:
                return
            stop.wait(0.2)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler)
    th.start()
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(8):
            run()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    # drop the first sample (taken while the loop ramped up)
    samples = samples[1:] if len(samples) > 2 else samples
    if not samples:
        return None, None
    return float(np.median([c for c, _ in samples])), float(np.median([p for _, p in samples]))


def mfma_ceiling(no_clock=False, iters=3000, reps=10):
    """What the int8 matrix cores sustain with no memory traffic: one wave per
    SIMD on every compute unit runs rns_probe_int8_mfma (32 MFMAs of 32x32x32
    per iteration, 16 accumulator chains) on random operand bytes and on zero
    bytes, timed with HIP events on the launch stream; the shader clock and
    socket power amd-smi reports while each runs back to back.  The dense
    peak assumes the full clock; the clock falls under the power limit with
    the switching of the operand bits, which the two data sets bracket."""
    import torch
    import exact_integer_gemm_amd as rg
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    ops = 2.0 * 32 ** 3 * 32 * iters * 4 * cus
    res = {"probe": "rns_probe_int8_mfma", "workgroups": cus, "iters": iters, "ops_per_launch": ops}
    for kind in ("random", "zero"):
        if kind == "random":
            src = torch.randint(-128, 128, (cus * 256 * 128,), dtype=torch.int8, device="cuda")
        else:
            src = torch.zeros(cus * 256 * 128, dtype=torch.int8, device="cuda")

        def run():
            rg.probe_int8_mfma(src, cus, iters)
        for _ in range(2):
            run()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        clk, pw = (None, None) if no_clock else gfx_clock_during(run)
        res[kind] = {"us": ms * 1e3, "TOPs": ops / (ms * 1e-3) / 1e12,
                     "frac_of_peak": ops / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS,
                     "clock_MHz": clk, "socket_power_W": pw}
    return res


def copy_probe():
    """A plain streaming kernel over 1 GiB (reads 1 GiB, writes 1 GiB), for counter scaling."""
    import torch
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)          # an elementwise streaming kernel
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n}), flush=True)


def enclosure_fp64(args):
    """The enclosure product on binary64 operands: A[1024,4096] @ B[4096,1024]
    of N(0,1) entries, (lo, hi) rounded outward.  One step is a whole
    mm_enclose call: the planner's reductions and their host synchronisation,
    the scaling into limbs, the exact product and the rounding."""
    import ctypes
    import torch
    import exact_integer_gemm_amd as rg
    from exact_integer_gemm_amd import enclose as EN

    rg.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    M, K, N = 1024, 4096, 1024
    rng = np.random.default_rng(3)
    A_h = rng.standard_normal((M, K))
    B_h = rng.standard_normal((K, N))
    A = torch.from_numpy(A_h).to(dev)
    B = torch.from_numpy(B_h).to(dev)
    lo, hi, ep = rg.mm_enclose(A, B, return_plan=True)
    ws = torch.empty(EN.workspace_size(ep, M, N, K), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        rg.mm_enclose(A, B, workspace=ws)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        lo, hi = rg.mm_enclose(A, B, workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # device stages of the same call, each timed alone (events on the stream)
    a_l, b_l, c_l = ep.limbs
    plan = rg.Plan._from_c(ep.c.plan)
    gws = rg.new_workspace(plan, M, N, K, False, dev)
    Ai = torch.empty((M, K, a_l), dtype=torch.int64, device=dev)
    Bi = torch.empty((K, N, b_l), dtype=torch.int64, device=dev)
    S = torch.empty((M, N, c_l), dtype=torch.int64, device=dev)
    stats = torch.empty(8, dtype=torch.int32, device=dev)
    sws = torch.empty(EN.FP_STATS_WS_BYTES, dtype=torch.uint8, device=dev)
    # the products and the reconstruction are the integer path's kernels on
    # the same planes: the split of the integer copies prepares them once
    rg.load().rns_fp64_to_limbs(A.data_ptr(), M * K, ep.fa, a_l, Ai.data_ptr(), stream.cuda_stream)
    rg.load().rns_fp64_to_limbs(B.data_ptr(), K * N, ep.fb, b_l, Bi.data_ptr(), stream.cuda_stream)
    rg.split(plan, Ai, Bi, gws, M=M)
    stages = {
        "stats_us": lambda: (EN.fp64_stats(A, stats[0:4], sws), EN.fp64_stats(B, stats[4:8], sws)),
        "mm_enclose_device_us": lambda: rg.load().rns_mm_enclose(
            ctypes.byref(ep.c), M, N, K, A.data_ptr(), B.data_ptr(), lo.data_ptr(), hi.data_ptr(),
            ws.data_ptr(), ws.numel(), stream.cuda_stream),
        "gemm_us": lambda: rg.residue_products(plan, M, N, K, gws),
        "reconstruct_us": lambda: rg.reconstruct(plan, M, N, K, gws, S),
        "round_us": lambda: rg.load().rns_round_outward(S.data_ptr(), M * N, c_l, ep.q, 64, lo.data_ptr(),
                                                        hi.data_ptr(), stream.cuda_stream),
    }
    out_st = {}
    for name, fn in stages.items():
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out_st[name] = e0.elapsed_time(e1) / 10 * 1e3
    gemm_ops = 2.0 * M * N * K * ep.n_primes
    gemm_tops = gemm_ops / (out_st["gemm_us"] * 1e-6) / 1e12
    width = rg.width_ulps(lo, hi)
    out = {
        "metric": "enclosure product rate (2MNK/s, lo <= A@B <= hi exactly)",
        "value": 2.0 * M * N * K / (ms_step * 1e-3), "unit": "ops/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "enclosure_fp64", "M": M, "N": N, "K": K, "operands": "binary64 N(0,1)",
                   "fa": ep.fa, "fb": ep.fb, "limbs": [a_l, b_l, c_l], "n_primes": ep.n_primes,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": gemm_tops, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": gemm_tops / PEAK_INT8_TOPS, "traffic": None,
                     "kernel": gemm_kernel_name(rg.layout(plan, M, N, K)["tile_config"], ep.n_primes, M, N)},
        "stages": out_st,
        "width_ulps_max": int(width.max()), "width_ulps_zero_frac": float((width == 0).float().mean()),
    }
    if not args.no_cpu_baseline:
        from oracle import enclose as E
        t = time.perf_counter()
        rows, cols = 2, 32
        rlo, rhi = E.enclose(A_h[:rows], B_h[:, :cols])
        dt = time.perf_counter() - t
        same = (np.array_equal(rlo.view(np.uint64), lo[:rows, :cols].cpu().numpy().view(np.uint64)) and
                np.array_equal(rhi.view(np.uint64), hi[:rows, :cols].cpu().numpy().view(np.uint64)))
        out["cpu_baseline"] = {"value": 2.0 * rows * cols * K / dt, "unit": "ops/s", "cores": 1,
                               "kind": "oracle", "bit_exact_sample": bool(same),
                               "sample": f"{rows}x{cols} entries of the product (all of K), Python Fraction "
                                         f"oracle ({dt:.1f} s)"}
    print(json.dumps(out), flush=True)


def solve_bench(args):
    """The exact rational solve A x = b (exact-solve): A [n, n] and b [n, c] of
    24-bit integers.  Times the GPU stages (batched inverse, lift) with events
    and the host reconstruction with a wall clock; one step is one solve."""
    import math
    import torch
    import exact_integer_gemm_amd as rg
    from exact_integer_gemm_amd import exact_solve as XS

    rg.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    n, c = args.n, args.rhs
    rng = np.random.default_rng(5)
    A_h = rng.integers(-2 ** 23, 2 ** 23, size=(n, n))
    b_h = rng.integers(-2 ** 23, 2 ** 23, size=(n, c))
    A = torch.from_numpy(A_h).to(dev)
    b = torch.from_numpy(b_h).to(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    times = {"inverse_ms": [], "lift_ms": [], "prep_during_lift_s": [], "reconstruct_s": [],
             "lowest_terms_s": [], "stages_total_s": []}
    native = XS.host_bigint_available()
    info = None
    for it in range(max(args.steps, 1) + 1):
        t_start = time.perf_counter()
        e0, e1 = ev(), ev()
        e0.record(stream)
        singular, ws = XS.batched_inverse(A)
        e1.record(stream)
        Nb, Db = XS._bounds(A_h, b_h)                  # on the host while the inverse runs, as solve() does
        sing = singular.cpu().tolist()
        sel = [i for i, v in enumerate(sing) if not v]
        moduli = [XS.ODD_PRIMES[i] for i in sel]
        p = XS.plan_from_moduli(moduli, n)
        planes = XS.inverse_planes(ws, n, sel)
        del ws
        P = math.prod(moduli)
        m = XS.lift_steps_for(P, Nb, Db)
        e2, e3 = ev(), ev()
        e2.record(stream)
        digits = XS.dixon_lift(p, A, b, planes, m)
        e3.record(stream)
        # the reconstruction's tables are built on the host while the lift runs, as solve() does
        t_tab = time.perf_counter()
        prep = XS.ReconstructionPrep(P, m, Db, dev, Nb, n * c) if native else None
        t_tab = time.perf_counter() - t_tab
        e3.synchronize()
        t_host = time.perf_counter()
        nums, den = XS.reconstruct_device(digits.reshape(m, n * c, -1), P, m, Nb, Db, prep)
        t_rec = time.perf_counter()
        XS.to_fractions(nums, den)
        t_end = time.perf_counter()
        if it == 0:
            info = {"primes": len(moduli), "steps": m, "log2_P": math.log2(P),
                    "denominator_bits": den.bit_length(),
                    "host_stage": ("p-adic values and D x mod P^m on the GPU, the sample's reconstruction on the host"
                                   if native else "Python integers")}
            # the identity A @ N == d * b on one column, in exact integers
            N0 = np.array(nums[0::c], dtype=object)
            ok = bool(np.array_equal(A_h.astype(object).dot(N0), den * b_h[:, 0].astype(object)))
            info["identity_A_N_eq_d_b"] = ok
            continue
        times["inverse_ms"].append(e0.elapsed_time(e1))
        times["lift_ms"].append(e2.elapsed_time(e3))
        times["prep_during_lift_s"].append(t_tab)
        times["reconstruct_s"].append(t_rec - t_host)
        times["lowest_terms_s"].append(t_end - t_rec)
        times["stages_total_s"].append(t_end - t_start)
    med = {k: float(np.median(v)) for k, v in times.items()}
    # the step itself: rg.solve(A, b) end to end, lowest-terms Fractions returned
    totals = []
    for _ in range(max(args.steps, 1)):
        t = time.perf_counter()
        x = rg.solve(A, b)
        totals.append(time.perf_counter() - t)
    med["total_s"] = float(np.median(totals))
    med["total_s_min"], med["total_s_max"] = float(min(totals)), float(max(totals))
    info["solution_is_fractions"] = bool(x is not None and isinstance(x[0][0], XS.Fraction))
    # the lift's products: 2 n n c per prime per step
    lift_ops = 2.0 * n * n * c * info["primes"] * info["steps"]
    out = {
        "metric": "exact rational solve wall time (rg.solve end to end: Dixon lift on the residue engine, "
                  "lowest-terms Fractions returned)",
        "value": med["total_s"], "unit": "s", "n_gpus": 1, "steps": args.steps, "warmup": 1,
        "ms_per_step": med["total_s"] * 1e3, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "solve", "n": n, "rhs": c, "entries": "uniform 24-bit", **info,
                   "parallelism": "single-gpu"},
        "stages": {**med, "lift_step_us": med["lift_ms"] * 1e3 / info["steps"],
                   "lift_product_TOPs": lift_ops / (med["lift_ms"] * 1e-3) / 1e12},
    }
    if not args.no_cpu_baseline:
        from oracle import dixon as D
        ns = min(n, 112)
        As = A_h[:ns, :ns].tolist()
        bs = b_h[:ns, :1].tolist()
        t = time.perf_counter()
        ref = D.solve_fraction(As, bs)
        dt = time.perf_counter() - t
        got = rg.solve(torch.tensor(As, dtype=torch.int64, device=dev), torch.tensor(bs, dtype=torch.int64,
                                                                                      device=dev))
        out["cpu_baseline"] = {"value": dt, "unit": "s", "cores": 1, "kind": "oracle",
                               "bit_exact_sample": got == ref,
                               "sample": f"Fraction Gaussian elimination of the leading {ns}x{ns} system "
                                         f"(one right-hand side); the oracle does not reach n = {n}"}
    print(json.dumps(out), flush=True)


def sliced_bench(args):
    """A product beyond the residue capacity: A[1024,1024] @ B[1024,1024] of full-range 4-limb
    entries (256-bit), through operand slices (four slice products of 3-limb slices)."""
    import torch
    from types import SimpleNamespace
    import exact_integer_gemm_amd as rg
    from exact_integer_gemm_amd import sliced as SL

    rg.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    M = N = K = 1024
    la = lb = 4
    rng = np.random.default_rng(6)
    A_h = rng.integers(0, 1 << 64, size=(M, K, la), dtype=np.uint64).view(np.int64)
    B_h = rng.integers(0, 1 << 64, size=(K, N, lb), dtype=np.uint64).view(np.int64)
    A = torch.from_numpy(A_h).to(dev)
    B = torch.from_numpy(B_h).to(dev)
    p = SL.sliced_plan(K, la, lb)
    ws = torch.empty(SL.workspace_size(p, M, N, K), dtype=torch.uint8, device=dev)
    C = torch.empty((M, N, p.out_limbs_min), dtype=torch.int64, device=dev)

    def run():
        SL.gemm_sliced(A, B, plan=p, workspace=ws, out=C)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / args.steps * 1e-3
    ops = 2.0 * M * N * K
    res_ops = p.products * ops * p.slice.n_primes
    out = {
        "metric": "exact int GEMM ops/s (2MNK/s), operands beyond the residue capacity",
        "value": ops / t, "unit": "ops/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": "sliced", "M": M, "N": N, "K": K, "limbs_in": [la, lb],
                   "limbs_out": p.out_limbs_min, "slices": [p.na, p.nb], "slice_limbs": [p.sa, p.sb],
                   "slice_primes": p.slice.n_primes, "entries": "full-range 256-bit",
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": res_ops / t / 1e12, "peak": 5000.0, "unit": "TOP/s",
                     "frac": res_ops / t / 1e12 / 5000.0, "traffic": None,
                     "kernel": "the whole call (slicing, four residue products with their splits and CRTs, the "
                               "shifted sum): a lower bound on the per-prime product rate"},
    }
    if not args.no_cpu_baseline:
        wl = SimpleNamespace(A=A_h, B=B_h, M=M, N=N, K=K)
        out["cpu_baseline"] = cpu_baseline(wl, p.slice, C, False, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.mfma_probe:
        print(json.dumps({"int8_mfma_ceiling": mfma_ceiling(args.no_clock)}), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.workload == "enclosure_fp64":
        enclosure_fp64(args)
        return
    if args.workload == "solve":
        solve_bench(args)
        return
    if args.workload == "sliced":
        sliced_bench(args)
        return

    import torch
    import exact_integer_gemm_amd as rg
    import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    rg.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    batched = args.workload == "dixon"
    if batched:
        plan = rg.plan_n(54)
        wl = W.make("dixon", primes=list(plan.primes))
        A_res = torch.from_numpy(wl.A_res).to(dev)
        A = None
    else:
        wl = W.make(args.workload)
        plan = rg.plan(wl.K, wl.a_bits, wl.b_bits)
        A = torch.from_numpy(wl.A).to(dev)
        A_res = None
    B = torch.from_numpy(wl.B).to(dev)
    M, N, K, n = wl.M, wl.N, wl.K, plan.n_primes
    lc = plan.out_limbs_min
    C = torch.empty((M, N, lc), dtype=torch.int64, device=dev)
    ws = rg.new_workspace(plan, M, N, K, batched, dev)
    tile_config = rg.layout(plan, M, N, K, batched)["tile_config"]
    if batched:
        dixon_bench(args, rg, wl, plan, A_res, B, C, ws, stream)
        return

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        rg.split(plan, A, B, ws, M=M)
        if evs is not None:
            evs[1].record(stream)
        rg.residue_products(plan, M, N, K, ws, A_res=A_res)
        if evs is not None:
            evs[2].record(stream)
        rg.reconstruct(plan, M, N, K, ws, C, batched=batched)
        if evs is not None:
            evs[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, events on the stream the kernels run on
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for s in range(args.steps):
        step(evs[s])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    st = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(3)] for e in evs])  # ms
    # means (the roofline divides by the average launch) and per-stage spread
    split_ms, gemm_ms, recon_ms = (float(x) for x in st.mean(axis=0))
    flags = rg.status(ws)
    digest = output_digest(args.workload, C)

    # the shader clock while the products run back to back (they run power
    # limited): the same peak scaled to that clock
    clk_mhz, power_w = (None, None) if args.no_clock else gfx_clock_during(
        lambda: rg.residue_products(plan, M, N, K, ws, A_res=A_res))

    # the matrix cores' own rate on random and zero operand bytes (no memory
    # traffic), next to which the products' fraction of the dense peak reads
    ceiling = mfma_ceiling(args.no_clock) if args.workload == "wide" else None

    # Garner reconstruction (same output) timed outside the step, for its
    # O(p^2) share next to the CRT that the step uses
    C2 = torch.empty_like(C)
    g_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    rg.reconstruct(plan, M, N, K, ws, C2, batched=batched, method="garner")
    g_ev[0].record(stream)
    g_reps = max(3, args.steps // 4)
    for _ in range(g_reps):
        rg.reconstruct(plan, M, N, K, ws, C2, batched=batched, method="garner")
    g_ev[1].record(stream)
    torch.cuda.synchronize()
    garner_ms = g_ev[0].elapsed_time(g_ev[1]) / g_reps
    same_as_garner = bool(torch.equal(C, C2))

    # the same step replayed from a HIP graph (G steps per graph): the
    # kernels' own pace, which the host's per-call dispatch hides on small
    # shapes.  `value` stays the eager step above.  Each of three further
    # replays follows eager work that overwrites C and is checked against
    # the eager output.
    eager_C = C.clone()
    G = 5
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(G):
            step()
    graph.replay()
    torch.cuda.synchronize()
    g_reps = max(2, args.steps // G)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(g_reps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / (g_reps * G)
    graph_same = True
    for _ in range(3):
        C.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        graph_same = graph_same and bool(torch.equal(C, eager_C))
    del graph

    # rates
    mnk2 = 2.0 * M * N * K
    logical = mnk2 * (n if batched else 1)        # the lift step has no single product
    value = logical / (ms_step * 1e-3)
    gemm_ops = mnk2 * n
    gemm_tops = gemm_ops / (gemm_ms * 1e-3) / 1e12
    la = 0 if batched else wl.la
    lb = wl.lb
    split_bytes = (0 if batched else M * K * (8 * la + n)) + K * N * (8 * lb + n)
    recon_bytes = M * N * (n + 8 * lc)
    gemm_min_bytes = n * (M * K + N * K + M * N)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "ops/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K, "limbs_in": [la, lb],
                   "limbs_out": lc, "n_primes": n, "parallelism": "single-gpu",
                   "note": wl.note},
        "roofline": {"bound": "mfma", "achieved": gemm_tops, "peak": PEAK_INT8_TOPS,
                     "unit": "TOP/s", "frac": gemm_tops / PEAK_INT8_TOPS,
                     "traffic": measured_traffic(args.workload),
                     "kernel": gemm_kernel_name(tile_config, n, M, N),
                     "algorithmic_ops_per_launch": gemm_ops,
                     "clock_MHz_during_products": clk_mhz, "socket_power_W_during_products": power_w,
                     "frac_at_measured_clock": (gemm_tops / (PEAK_INT8_TOPS * clk_mhz / 2400.0)
                                                if clk_mhz else None),
                     "int8_mfma_ceiling": ceiling,
                     "frac_of_random_operand_ceiling": (gemm_tops / ceiling["random"]["TOPs"]
                                                        if ceiling else None)},
        "output": digest,
        "stages": {
            "split_us_spread": spread(st[:, 0]), "products_us_spread": spread(st[:, 1]),
            "reconstruct_us_spread": spread(st[:, 2]),
            "split_us": split_ms * 1e3, "split_GBps": split_bytes / (split_ms * 1e-3) / 1e9,
            "gemm_us": gemm_ms * 1e3, "gemm_TOPs": gemm_tops,
            "gemm_min_GBps": gemm_min_bytes / (gemm_ms * 1e-3) / 1e9,
            "reconstruct_us": recon_ms * 1e3, "reconstruct_GBps": recon_bytes / (recon_ms * 1e-3) / 1e9,
            "reconstruct_share": recon_ms / (split_ms + gemm_ms + recon_ms),
            "reconstruct_method": "crt_rounded_quotient_mfma",
            "garner_us": garner_ms * 1e3, "garner_GBps": recon_bytes / (garner_ms * 1e-3) / 1e9,
            "garner_share_if_used": garner_ms / (split_ms + gemm_ms + garner_ms),
            "garner_bit_identical": same_as_garner,
            "hbm_peak_GBps": PEAK_HBM_GBPS,
            "graph_step_us": graph_ms * 1e3, "graph_steps_per_replay": G,
            "graph_output_equals_eager": graph_same,
        },
        "status_flags": flags,
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, plan, C, batched, args.cpu_seconds)
        if args.workload == "square":
            out["cpu_baseline_one_thread"] = cpu_one_thread(args.workload, C.shape[-1], 64, M, N, K)
    print(json.dumps(out), flush=True)


def dixon_bench(args, rg, wl, plan, A_res, B, C, ws, stream):
    """The Dixon-lift step as one rns_gemm_batched_residue call (one kernel:
    the products on r's bytes and the reconstruction).  Steps run back to
    back on one stream; they are captured G at a time in a HIP graph and
    replayed, so that host dispatch does not pace a step of some tens of
    microseconds (G divides the step count; every step is a full call)."""
    import torch
    M, N, K, n = wl.M, wl.N, wl.K, plan.n_primes
    lc = C.shape[-1]

    def call():
        rg.gemm_batched_residue(plan, A_res, B, out=C, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / args.steps
    eager_out = C.clone()

    G = max(d for d in range(1, 26) if args.steps % d == 0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(G):
            call()
    for _ in range(max(1, args.warmup // G)):
        g.replay()
    torch.cuda.synchronize()
    reps = args.steps // G
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for s in range(reps):
        g.replay()
        evs[s + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[s].elapsed_time(evs[s + 1]) / G for s in range(reps)]
    ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    same_as_eager = bool(torch.equal(C, eager_out))
    digest = output_digest(args.workload, C)

    # cold steps: before each, a read pass over 1 GiB (a max reduction) evicts
    # the 256 MB last-level cache (MALL) and the L2s, leaving clean lines.
    # Everything is queued ahead, so the GPU never idles between the flush and
    # the call; events around the call alone time it.
    flush = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")
    sink = torch.zeros((), dtype=torch.int32, device="cuda")
    n_cold = min(args.steps, 40)
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_cold)]
    torch.cuda.synchronize()
    for c0, c1 in cev:
        sink.copy_(flush.max())
        c0.record(stream)
        call()
        c1.record(stream)
    torch.cuda.synchronize()
    cold = [c0.elapsed_time(c1) for c0, c1 in cev]
    del flush, sink

    logical = 2.0 * M * N * K * n
    step_bytes = n * M * K + K * N * 8 * B.shape[-1] + M * N * 8 * lc
    out = {
        "metric": METRIC, "value": logical / (ms_step * 1e-3), "unit": "ops/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K, "n_primes": n, "limbs_out": lc,
                   "parallelism": "single-gpu", "note": wl.note,
                   "launch": "one rns_gemm_batched_residue call per step, G steps per HIP graph replay",
                   "steps_per_graph": G},
        "roofline": {"bound": "hbm", "achieved": step_bytes / (ms_step * 1e-3) / 1e9, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                     "traffic": None, "scope": "whole step (one kernel)",
                     "algorithmic_bytes_per_step": step_bytes,
                     # the kernel's int8 products: nine 16-column blocks (the eight bytes of r
                     # and the row sums) per product row, for every prime
                     "int8_mfma_ops_per_step": 2.0 * n * M * 9 * 16 * K,
                     "int8_mfma_frac": 2.0 * n * M * 9 * 16 * K / (ms_step * 1e-3) / 1e12 / PEAK_INT8_TOPS},
        "output": digest,
        "stages": {"step_us_spread_per_replay": spread(per), "eager_call_us": eager_ms * 1e3,
                   "cold_step_us": spread(cold),
                   "graph_output_equals_eager": same_as_eager},
        "status_flags": rg.status(ws),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, plan, C, True, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_one_thread(workload, lc, rows, M, N, K):
    """The C oracle with one OpenMP thread on the first `rows` rows of the
    workload (a child process: the thread count is fixed when the library
    starts), next to the all-cores figure."""
    import subprocess
    code = ("import time, workloads as W; from oracle import cgemm; "
            f"wl = W.make({workload!r}); cgemm.build(); "
            f"t = time.perf_counter(); cgemm.gemm(wl.A[:{rows}], wl.B, {lc}); print(time.perf_counter() - t)")
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300,
                           cwd=os.path.dirname(os.path.abspath(__file__)))
        dt = float(r.stdout.strip().splitlines()[-1])
    except Exception as e:              # reported, never fatal to the benchmark line
        return {"error": str(e)[:200]}
    return {"value": 2.0 * rows * N * K / dt, "unit": "ops/s", "cores": 1, "kind": "oracle",
            "sample": f"first {rows} of {M} rows of C (all of B), C schoolbook oracle, one thread",
            "seconds": dt}


def cpu_baseline(wl, plan, C_gpu, batched, target_s):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import torch
    from oracle import cgemm
    from oracle import oracle as O

    if batched:
        # the lift step: numpy int64 products per prime + textbook CRT, on a
        # sample of rows of the residue planes
        rows = 16
        t = time.perf_counter()
        X = O.residue_gemm_via_crt(wl.A_res[:, :rows], wl.B[..., 0], list(plan.primes))
        dt = time.perf_counter() - t
        got = O.decode_array(C_gpu[:rows].cpu().numpy())
        ops = 2.0 * rows * wl.N * wl.K * plan.n_primes
        return {"value": ops / dt, "unit": "ops/s", "cores": 1, "kind": "oracle",
                "sample": f"{rows} of {wl.M} rows, all 54 primes (numpy int64 products, Python CRT)",
                "seconds": dt, "bit_exact_sample": bool(np.array_equal(got, X))}
    cgemm.build()
    lc = C_gpu.shape[-1]

    def timed(rows):
        t = time.perf_counter()
        ref = cgemm.gemm(wl.A[:rows], wl.B, lc)
        return time.perf_counter() - t, ref

    # grow the sample until it takes about target_s (a few probes, capped at all rows)
    rows = min(4, wl.M)
    dt, ref = timed(rows)
    while dt < 0.5 * target_s and rows < wl.M:
        rows = int(min(wl.M, max(rows + 1, round(rows * target_s / max(dt, 1e-6)))))
        dt, ref = timed(rows)
    got = C_gpu[:rows].cpu().numpy()
    ops = 2.0 * rows * wl.N * wl.K
    return {"value": ops / dt, "unit": "ops/s", "cores": cgemm.threads_used(), "kind": "oracle",
            "sample": f"first {rows} of {wl.M} rows of C (all of B), C schoolbook oracle",
            "seconds": dt, "bit_exact_sample": bool(np.array_equal(got, ref))}


if __name__ == "__main__":
    main()
