#!/usr/bin/env python3
"""Benchmark: emulated FP64 GEMM (Ozaki Scheme II on int8 matrix cores).

One step = one ``ozgemm_dgemm`` call: scale, residue, s int8 GEMMs with the
fused product re-reduction, CRT reconstruction and unscaling, on inputs that
are already resident in HBM.  Default workload: m = n = q = 8192, s = 14,
HPL-like inputs with phi = 1 (seed 0).

Prints ONE JSON line with the throughput (2 m n q / time, in emulated FP64
TFLOPS), a roofline object for the dominant kernel (the int8 GEMM, priced
against the MI355X dense int8 peak), the CPU oracle timed on a bounded
sample of the same workload, and as context the rate a register-only MFMA
loop sustains under the power limit, correct bits, and the native FP64
GEMM (torch.matmul) on the same inputs.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 matrix peak (5.0 POP/s)
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E peak


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--m", type=int, default=8192)
    p.add_argument("--n", type=int, default=8192)
    p.add_argument("--q", type=int, default=8192)
    p.add_argument("--s", type=int, default=14)
    p.add_argument("--phi", type=float, default=1.0)
    p.add_argument("--bound", choices=["conservative", "fast", "accu"], default="conservative",
                   help="bit budget: the k of the Ozaki II notes section 5, or OS II-fast / OS II-accu (section 9)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--panels", type=int, default=0,
                   help="column panels of the CRT/product pipeline (ozgemm_set_panels): 0 or 1 off, P >= 2 forced")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target duration of the oracle sample")
    p.add_argument("--cpu-workers", type=int, default=0, help="oracle worker processes (default: host CPUs, <= 16)")
    p.add_argument("--settle-seconds", type=float, default=2.0,
                   help="untimed steady-state window after the warmup calls, timed per call with HIP events")
    p.add_argument("--bits-entries", type=int, default=4096, help="sampled output entries for the correct bits")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-accuracy", action="store_true")
    p.add_argument("--no-native", action="store_true", help="skip the native FP64 matmul context figures")
    p.add_argument("--no-ceiling", action="store_true", help="skip the matrix-core rate probe")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="also run one plain device copy of this many bytes (calibrates HBM byte counters)")
    return p.parse_args()


def kernel_hash() -> str:
    """Hash of the int8 GEMM kernel's sources (the same as the one stored
    with the counter record)."""
    from fp64_gemm_emulation_ozii_amd.profiling import kernel_sha
    return kernel_sha()


def traffic_record(workload: str):
    """HBM bytes per GEMM launch from the committed counter summary
    (profiles/traffic.json), or None when it is absent or was taken on a
    different GEMM kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        ent = rec.get(workload)
        if not ent or ent.get("kernel_sha") != kernel_hash():
            return None
        v = ent.get("gemm_hbm_bytes_per_launch")
        return None if v is None else int(v)
    except Exception:
        return None


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, run as it stands, in worker processes on the
# host's cores (each worker evaluates oracle.ozaki2.dgemm_block on a block of
# rows of the sampled output block; BLAS in each worker is single-threaded)
# ---------------------------------------------------------------------------
_W = {}


def _oracle_worker_init(Bcols, s, bound):
    _W["B"], _W["s"], _W["bound"] = Bcols, s, bound


def _oracle_worker_block(Arows):
    from oracle import ozaki2 as oz
    import numpy as np
    B = _W["B"]
    return oz.dgemm_block(Arows, B, _W["s"], np.arange(Arows.shape[0]), np.arange(B.shape[1]), bound=_W["bound"])


def mfma_loop_ceiling(L, dev, target_ms: float = 200.0, runs: int = 3):
    """Sustained int8 rate of a register-only MFMA loop on every CU
    (ozgemm_mfma_ceiling), timed with HIP events: the median of `runs` runs
    of about target_ms each."""
    import torch
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(4 * blocks, dtype=torch.int32, device=dev)

    def timed(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        L.ozgemm_mfma_ceiling(blocks, steps, 1, sink)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    steps = 16384
    timed(steps)                     # first launch: code load and clock ramp
    ms = timed(steps)
    steps = max(16384, min(1 << 26, int(steps * target_ms / max(ms, 1e-3))))
    times = [timed(steps) for _ in range(runs)]
    med = statistics.median(times)
    ops = float(blocks) * 4 * steps * 2**20
    tops = ops / (med * 1e-3) / 1e12
    return {"tops": round(tops, 2), "ms": round(med, 3), "blocks": blocks, "steps": steps,
            "instruction": "v_mfma_i32_16x16x64_i8", "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}


def host_cpus() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(A, B, s, q, target_s, Cg_full_getter, bound="conservative", workers=0):
    """Time the oracle on a block of output entries of the same workload,
    spread over `workers` processes (default: the host's CPUs, at most 16)."""
    import multiprocessing as mp
    import numpy as np
    m, n = A.shape[0], B.shape[1]
    cpus = host_cpus()
    W = workers if workers > 0 else max(1, min(16, cpus))
    rng = np.random.default_rng(7)
    ncols = min(n, 256)
    cols = np.sort(rng.choice(n, size=ncols, replace=False))
    Bc = np.ascontiguousarray(B[:, cols])
    blas_env = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in blas_env}
    for k in blas_env:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")  # fresh interpreters that never touch the GPU
        with ctx.Pool(W, initializer=_oracle_worker_init, initargs=(Bc, s, bound)) as pool:
            # calibrate with blocks of 4 and then 20 rows per worker: a block
            # costs a fixed part (B's residues for the sampled columns) plus a
            # part per row; size one block per worker for about target_s
            perm = rng.permutation(m)

            def timed_round(nrows):
                blocks = [np.sort(perm[(nrows * w) % m:(nrows * w) % m + nrows]) for w in range(W)]
                t0 = time.perf_counter()
                pool.map(_oracle_worker_block, [np.ascontiguousarray(A[b, :]) for b in blocks], chunksize=1)
                return time.perf_counter() - t0

            timed_round(1)  # workers import the oracle
            t4, t20 = timed_round(4), timed_round(20)
            per_row = max((t20 - t4) / 16.0, 1e-6)
            fixed = max(t4 - 4 * per_row, 0.0)
            rows_per_worker = int(max(8, min(-(-m // W), (target_s - fixed) / per_row)))
            total = min(m, rows_per_worker * W)
            rows = np.sort(perm[:total])
            blocks = np.array_split(rows, W)
            t0 = time.perf_counter()
            parts = pool.map(_oracle_worker_block, [np.ascontiguousarray(A[b, :]) for b in blocks], chunksize=1)
            dt = time.perf_counter() - t0
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    ref = np.concatenate(parts, axis=0)
    entries = ref.shape[0] * ref.shape[1]
    Cg = Cg_full_getter(rows, cols)
    exact = int(np.sum(Cg.view(np.uint64) == ref.view(np.uint64)))
    return {
        "value": 2.0 * q * entries / dt / 1e12,
        "unit": "TFLOPS",
        "cores": W,
        "kind": "oracle",
        "sample": f"{len(rows)}x{len(cols)} output block (random rows and columns) of the same workload, "
                  f"{dt:.1f} s wall on {W} worker processes (one oracle.ozaki2.dgemm_block per row block, "
                  f"single-threaded BLAS each)",
        "seconds": dt,
        "host_cpus": cpus,
        "nproc": os.cpu_count(),
        "extrapolated_full_seconds": round(dt * m * n / entries, 1),  # the whole output, extrapolated
        "parity_entries": entries,
        "parity_bit_exact": exact,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the emulated GEMM shards by output tiles, see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from fp64_gemm_emulation_ozii_amd import ozgemm as L
    from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like

    m, n, q, s, phi = args.m, args.n, args.q, args.s, args.phi
    workload = f"ozaki2_dgemm_{m}x{n}x{q}_s{s}_phi{phi:g}" + ("" if args.bound == "conservative" else f"_{args.bound}")
    A, B = hpl_like(m, q, n, phi, seed=args.seed)
    dev = torch.device("cuda:0")
    Ad = torch.from_numpy(np.ascontiguousarray(A.T)).to(dev)   # column-major A, lda = m
    Bd = torch.from_numpy(np.ascontiguousarray(B.T)).to(dev)   # column-major B, ldb = q
    Cd = torch.empty((n, m), dtype=torch.float64, device=dev)  # column-major C, ldc = m
    stream = torch.cuda.current_stream()
    L.ozgemm_config(s, m, n, q, stream=stream)
    if args.bound != "conservative":
        L.ozgemm_set_bound(L.OZGEMM_BOUND_FAST if args.bound == "fast" else L.OZGEMM_BOUND_ACCU)
    L.ozgemm_set_panels(args.panels)

    def call():
        L.ozgemm_dgemm(m, n, q, Ad, m, Bd, q, Cd, m, s)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes // 8, dtype=torch.float64, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Steady state: the part runs under a power limit, and a short burst on a
    # cool chip runs faster than the sustained rate.  Keep it busy for at
    # least settle_seconds (calls timed one by one with HIP events on the
    # library's stream), then time the K steps right after.
    steady = None
    if args.settle_seconds > 0:
        L.ozgemm_timing(True)
        t0 = time.perf_counter()
        ncalls = 0
        while True:
            batch = max(1, min(256, 4096 - ncalls))
            for _ in range(batch):
                call()
            ncalls += batch
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= args.settle_seconds or ncalls >= 4096:
                break
        wall = time.perf_counter() - t0
        per_call = L.ozgemm_phase_calls()
        L.ozgemm_timing(False)
        tot = sorted(sum(c) for c in per_call)
        gem = sorted(c[2] for c in per_call)
        steady = {
            "seconds": round(wall, 3), "calls": ncalls,
            "ms_per_call_median": round(statistics.median(tot), 4),
            "ms_per_call_mean": round(statistics.fmean(tot), 4),
            "gemm_ms_median": round(statistics.median(gem), 4),
            "gemm_ms_mean": round(statistics.fmean(gem), 4),
            "tflops_at_median": round(2.0 * m * n * q / (statistics.median(tot) * 1e-3) / 1e12, 3),
            "gemm_peak_frac_at_median": round(2.0 * s * m * n * q / (statistics.median(gem) * 1e-3) / 1e12
                                              / INT8_PEAK_TOPS, 4),
        }

    L.ozgemm_timing(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per_call = L.ozgemm_phase_calls()
    L.ozgemm_timing(False)

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tflops = 2.0 * m * n * q / (ms_per_step * 1e-3) / 1e12
    per = [statistics.fmean(c[p] for c in per_call) for p in range(4)]
    totals = [sum(c) for c in per_call]
    gemm_ms = per[2]
    int8_ops = 2.0 * s * m * n * q
    achieved = int8_ops / (gemm_ms * 1e-3) / 1e12
    mp, np_, qp = L.ozgemm_plane_dims(m, n, q)
    b_one_pass = args.bound == "conservative" and L.OZGEMM_ONE_PASS_Q_MIN <= q <= L.OZGEMM_ONE_PASS_Q_MAX

    out = {
        "metric": "emulated-FP64 TFLOPS (2mnq/t) at 8192^3, s=14; INT8 MFMA peak fraction",
        "value": round(tflops, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_event_median": round(statistics.median(totals), 4),
        "ms_per_step_event_mean": round(statistics.fmean(totals), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": workload, "m": m, "n": n, "q": q, "s": s, "phi": phi, "seed": args.seed,
                   "output_dtype": "f64", "layout": "column-major NN", "bit_budget": args.bound,
                   "panels": args.panels},
        "roofline": {
            "bound": "mfma",
            "kernel": "gemm_i8_kernel",
            "achieved": round(achieved, 2),
            "peak": INT8_PEAK_TOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / INT8_PEAK_TOPS, 4),
            "traffic": traffic_record(workload),
            "algorithmic_ops_per_launch": int8_ops,
        },
        "phases_ms": {"scale": round(per[0], 4), "residue": round(per[1], 4), "gemm": round(per[2], 4),
                      "crt": round(per[3], 4)},
        "gemm_ms_median": round(statistics.median(c[2] for c in per_call), 4),
        "steady_state": steady,
        "int8_tops_end_to_end": round(int8_ops / (ms_per_step * 1e-3) / 1e12, 2),
        "int8_peak_frac_end_to_end": round(int8_ops / (ms_per_step * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
        "memory_phases_GBs": {
            # B is read by the scale phase only when its exponents are not
            # taken in the residue pass (OS II-fast, or q outside the one-pass range)
            "scale": round(8.0 * (m * q + (0 if b_one_pass else q * n)) / (per[0] * 1e-3) / 1e9, 1),
            "residue": round((8.0 + s) * (m * q + q * n) / (per[1] * 1e-3) / 1e9, 1),
            "crt": round((s + 8.0) * m * n / (per[3] * 1e-3) / 1e9, 1),
        },
    }

    # The int8 rate the matrix cores sustain on their own under the power
    # limit (register-only MFMA loop in the product kernel's issue order,
    # about 200 ms per run on a chip that is already warm), beside the
    # clock-rate figure the roofline uses
    if not args.no_ceiling:
        ceil = mfma_loop_ceiling(L, dev)
        out["mfma_loop_ceiling"] = ceil
        out["gemm_frac_of_mfma_loop_ceiling"] = round(achieved / ceil["tops"], 4)

    def block_getter(rows, cols):
        r = torch.from_numpy(rows).to(dev)
        c = torch.from_numpy(cols).to(dev)
        return Cd[c][:, r].cpu().numpy().T

    if not args.no_accuracy:
        from fp64_gemm_emulation_ozii_amd.accuracy import correct_bits_many
        from fp64_gemm_emulation_ozii_amd.synthetic import sample_entries
        ri, ci = sample_entries(m, n, args.bits_entries, seed=3)
        Cg = Cd.T[torch.from_numpy(ri).to(dev), torch.from_numpy(ci).to(dev)].cpu().numpy()
        out["correct_bits"] = round(correct_bits_many(Cg, A, B, ri, ci), 2)
        native = (torch.from_numpy(A[ri, :]).to(dev) * torch.from_numpy(B[:, ci].T.copy()).to(dev)).sum(1)
        out["correct_bits_native_fp64_dot"] = round(correct_bits_many(native.cpu().numpy(), A, B, ri, ci), 2)
        out["correct_bits_entries"] = int(len(ri))
        if not args.no_native:
            # context: the native FP64 GEMM of the same inputs (torch.matmul,
            # the vendor BLAS), its time and its correct bits on the same entries
            Cn = torch.empty((n, m), dtype=torch.float64, device=dev)   # C^T = B^T A^T, row-major
            torch.matmul(Bd, Ad, out=Cn)
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
            for e0, e1 in evs:
                e0.record()
                torch.matmul(Bd, Ad, out=Cn)
                e1.record()
            torch.cuda.synchronize()
            nms = statistics.median(e0.elapsed_time(e1) for e0, e1 in evs)
            Cv = Cn[torch.from_numpy(ci).to(dev), torch.from_numpy(ri).to(dev)].cpu().numpy()
            out["native_fp64_matmul"] = {
                "ms": round(nms, 4), "tflops": round(2.0 * m * n * q / (nms * 1e-3) / 1e12, 3),
                "correct_bits": round(correct_bits_many(Cv, A, B, ri, ci), 2), "calls": len(evs),
            }
            del Cn

    if not args.no_cpu_baseline and args.bound == "accu":
        # OS II-accu's row and column bit counts depend on all of A and B, so a
        # block of the oracle is not the oracle on the block's rows and columns
        out["cpu_baseline"] = None
    elif not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(A, B, s, q, args.cpu_seconds, block_getter, args.bound, args.cpu_workers)
    L.ozgemm_free()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
