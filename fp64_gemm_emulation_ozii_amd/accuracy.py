"""Accuracy and phase-time measurement of the emulated DGEMM.

Correct bits of an output entry are -log2(|C_ij - (AB)_ij| / (|A||B|)_ij);
over a set of entries the worst one counts.  This is the componentwise
measure behind the error bound of the Ozaki II notes (§5: the truncation
error of A' and B' relative to |A||B|), and 64 means exact everywhere.
correct_bits forms (AB)_ij and (|A||B|)_ij exactly in integer arithmetic
(a few entries); correct_bits_many uses compensated dot products kept
unrounded, whose error is far below what the measure resolves, for
thousands of entries (the sweep and the benchmark use it).

Command line (runs on the GPU)::

    python -m fp64_gemm_emulation_ozii_amd.accuracy --m 1024 --n 1024 --q 1024 \
        --s 8,10,12,14,16,18 --phi 0.5 [--entries 1024] [--out table.json]

prints one JSON object per (method, s or k, phi) with the correct bits of the
emulation and of the native FP64 dot products on the same entries, and the
time of each phase in milliseconds (Scheme II: scale, residue, GEMM, CRT;
Scheme I: split, products, accumulation).  ``--methods ozaki2,scheme1-rn,
scheme1-hybrid --k 4,5,6,7,8`` compares the two schemes on the same inputs;
``ozaki2-fast`` and ``ozaki2-accu`` are Scheme II under the OS II-fast and
OS II-accu bit budgets (§9).
"""
from __future__ import annotations

import argparse
import json
import math
import sys
from fractions import Fraction

import numpy as np


def _int_terms(v: np.ndarray):
    """Each double as (integer mantissa, exponent): v = mant * 2^expo."""
    mant, expo = np.frexp(np.asarray(v, dtype=np.float64))
    return (mant * float(1 << 53)).astype(np.int64), expo.astype(np.int64) - 53


def _exact_sum_products(a: np.ndarray, b: np.ndarray):
    """sum_l a_l b_l exactly, as (N, p) meaning N * 2^p."""
    ma, ea = _int_terms(a)
    mb, eb = _int_terms(b)
    nz = (ma != 0) & (mb != 0)
    if not nz.any():
        return 0, 0
    ma, ea, mb, eb = ma[nz], ea[nz], mb[nz], eb[nz]
    ex = ea + eb
    p = int(ex.min())
    total = 0
    for x, y, e in zip(ma.tolist(), mb.tolist(), (ex - p).tolist()):
        total += (x * y) << e
    return total, p


def entry_error(c: float, a: np.ndarray, b: np.ndarray):
    """|c - a.b| / (|a|.|b|) as a Fraction (None when |a|.|b| = 0)."""
    N, p = _exact_sum_products(a, b)
    D, pd = _exact_sum_products(np.abs(a), np.abs(b))
    if D == 0:
        return None
    exact = Fraction(N) * Fraction(2) ** p
    denom = Fraction(D) * Fraction(2) ** pd
    if not math.isfinite(c):
        return Fraction(1 << 64)
    return abs(Fraction(c) - exact) / denom


def correct_bits(values, A: np.ndarray, B: np.ndarray, rows, cols) -> float:
    """Worst-entry correct bits of values[k] = C[rows[k], cols[k]]."""
    worst = Fraction(0)
    for c, i, j in zip(values, rows, cols):
        err = entry_error(float(c), A[i, :], B[:, j])
        if err is not None and err > worst:
            worst = err
    return 64.0 if worst == 0 else -math.log2(float(worst))


def _two_sum_err(a, b, s):
    """Error of s = fl(a + b), exactly (Knuth's TwoSum)."""
    bb = s - a
    return (a - (s - bb)) + (b - bb)


def _split(a):
    """Dekker's split a = hi + lo with hi holding the top 26 bits (|a| < 2^995)."""
    t = 134217729.0 * a  # 2^27 + 1
    hi = t - (t - a)
    return hi, a - hi


def _two_prod_err(a, b, p):
    """Error of p = fl(a b), exactly (Dekker's TwoProduct, no fma), barring
    underflow."""
    ah, al = _split(a)
    bh, bl = _split(b)
    return ((ah * bh - p) + ah * bl + al * bh) + al * bl


def compensated_dots(a: np.ndarray, b: np.ndarray):
    """Row-wise dot products of a and b (E x q) as unevaluated pairs (hi, lo):
    TwoProduct on every term, then a pairwise TwoSum tree, with the product
    and addition errors summed in ordinary float64.  |hi + lo - a.b| is of
    order (log2 q + q 2^-53) 2^-106 |a|.|b| (Ogita, Rump and Oishi, 2005, for
    the same error-free transformations), far below the 2^-60 a correct-bit
    figure needs.  Entries must be scaled so that no product underflows or
    overflows (|a|, |b| < 1 and not too small, see correct_bits_many)."""
    p = a * b
    lo = _two_prod_err(a, b, p).sum(axis=1)
    x = p
    while x.shape[1] > 1:
        if x.shape[1] % 2:
            x = np.concatenate([x, np.zeros((x.shape[0], 1))], axis=1)
        u, v = x[:, 0::2], x[:, 1::2]
        sm = u + v
        lo = lo + _two_sum_err(u, v, sm).sum(axis=1)
        x = sm
    return x[:, 0], lo


def correct_bits_many(values, A: np.ndarray, B: np.ndarray, rows, cols, chunk: int = 256):
    """Worst-entry correct bits of values[k] = C[rows[k], cols[k]] for
    thousands of entries: the reference (AB)_ij is a compensated dot product
    kept unrounded (see compensated_dots), after scaling row i of A and column
    j of B by exact powers of two so that their maxima lie in [1/2, 1).  The
    measure |C - AB| / (|A||B|) does not change under that scaling.  Entries
    whose scaled terms fall below 2^-1000 add under 2^-1000 to (|A||B|)_ij,
    so dropping them to zero by underflow moves the figure by nothing
    measurable.  Non-finite values count as wrong (0 bits)."""
    vals = np.asarray(values, dtype=np.float64)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    worst = 0.0
    for c0 in range(0, len(rows), chunk):
        r, c, v = rows[c0:c0 + chunk], cols[c0:c0 + chunk], vals[c0:c0 + chunk]
        a = np.asarray(A[r, :], dtype=np.float64)
        b = np.asarray(B[:, c].T, dtype=np.float64)
        _, ea = np.frexp(np.max(np.abs(a), axis=1))
        _, eb = np.frexp(np.max(np.abs(b), axis=1))
        with np.errstate(under="ignore"):
            a = np.ldexp(a, -ea[:, None])
            b = np.ldexp(b, -eb[:, None])
            vs = np.ldexp(v, -(ea + eb))
            hi, lo = compensated_dots(a, b)
            den = np.sum(np.abs(a * b), axis=1)
            err = np.abs((vs - hi) - lo)
        ok = den > 0
        bad = ok & ~np.isfinite(vs)
        if bad.any():
            return 0.0
        rel = np.where(ok, err / np.where(ok, den, 1.0), 0.0)
        worst = max(worst, float(rel.max(initial=0.0)))
    return 64.0 if worst == 0 else min(64.0, -math.log2(worst))


def _parse_list(text: str, conv):
    return [conv(x) for x in text.split(",") if x.strip()]


def _runs(s_list, k_list, methods):
    """(method, parameter) pairs: Scheme II over s, Scheme I variants over k."""
    out = []
    for meth in methods:
        if meth in ("ozaki2", "ozaki2-fast", "ozaki2-accu"):
            out += [(meth, s) for s in s_list]
        elif meth in ("scheme1-rn", "scheme1-hybrid"):
            out += [(meth, k) for k in k_list]
        else:
            raise SystemExit(f"unknown method {meth}")
    return out


def run_sweep(m, n, q, s_list, phi_list, entries, seed, repeats, k_list=(), methods=("ozaki2",)):
    import torch

    from . import ozgemm as L
    from .synthetic import hpl_like

    dev = torch.device("cuda:0")
    from .synthetic import sample_entries
    rows, cols = sample_entries(m, n, entries, seed=12345)
    runs = _runs(s_list, k_list, methods)
    results = []
    for phi in phi_list:
        A, B = hpl_like(m, q, n, phi, seed=seed)
        Ad = torch.from_numpy(np.ascontiguousarray(A.T)).to(dev)
        Bd = torch.from_numpy(np.ascontiguousarray(B.T)).to(dev)
        Cd = torch.empty((n, m), dtype=torch.float64, device=dev)
        native = (torch.from_numpy(A[rows, :]).to(dev) * torch.from_numpy(B[:, cols].T.copy()).to(dev)).sum(1)
        native_bits = correct_bits_many(native.cpu().numpy(), A, B, rows, cols)
        s_max = max([p for meth, p in runs if meth.startswith("ozaki2")] or [1])
        need1 = max([L.ozgemm_scheme1_workspace_bytes(m, n, q, p, L.OZGEMM_S1_RN if meth == "scheme1-rn"
                                                       else L.OZGEMM_S1_HYBRID)
                     for meth, p in runs if not meth.startswith("ozaki2")] or [0])
        ws = torch.empty(max(L.ozgemm_workspace_bytes(m, n, q, s_max), need1), dtype=torch.uint8, device=dev)
        L.ozgemm_config(s_max, m, n, q, stream=torch.cuda.current_stream(), workspace=ws)

        def call(meth, p):
            if meth.startswith("ozaki2"):
                L.ozgemm_set_bound({"ozaki2-fast": L.OZGEMM_BOUND_FAST, "ozaki2-accu": L.OZGEMM_BOUND_ACCU}.get(
                    meth, L.OZGEMM_BOUND_CONSERVATIVE))
                L.ozgemm_dgemm(m, n, q, Ad, m, Bd, q, Cd, m, p)
            else:
                v = L.OZGEMM_S1_RN if meth == "scheme1-rn" else L.OZGEMM_S1_HYBRID
                L.ozgemm_scheme1_dgemm(m, n, q, Ad, m, Bd, q, Cd, m, p, v)

        for meth, p in runs:
            call(meth, p)  # warm-up
            torch.cuda.synchronize()
            L.ozgemm_timing(True)
            for _ in range(repeats):
                call(meth, p)
            torch.cuda.synchronize()
            phase_ms, calls = L.ozgemm_phase_ms()
            L.ozgemm_timing(False)
            per = [x / max(calls, 1) for x in phase_ms]
            Cs = Cd.T[torch.from_numpy(rows).to(dev), torch.from_numpy(cols).to(dev)].cpu().numpy()
            rec = {"method": meth, "m": m, "n": n, "q": q, "phi": phi}
            if meth.startswith("ozaki2"):
                rec.update({"s": p, "k": L.ozgemm_kbits(p, q), "int8_gemms": p})
                names = ("scale", "residue", "gemm", "crt")
            else:
                v = L.OZGEMM_S1_RN if meth == "scheme1-rn" else L.OZGEMM_S1_HYBRID
                rec.update({"slices": p, "beta": L.ozgemm_scheme1_beta(q), "int8_gemms": p * (p + 1) // 2,
                            "int32_outputs": L.ozgemm_scheme1_outputs(p, v, q)})
                names = ("scale", "split", "products", "accumulate")
            rec.update({
                "correct_bits": round(correct_bits_many(Cs, A, B, rows, cols), 2),
                "correct_bits_native_fp64": round(native_bits, 2),
                "entries": int(len(rows)),
                "phases_ms": {nm: round(x, 4) for nm, x in zip(names, per)},
                "total_ms": round(sum(per), 4),
                "fp64_tflops": round(2.0 * m * n * q / (sum(per) * 1e-3) / 1e12, 2),
            })
            print(json.dumps(rec), flush=True)
            results.append(rec)
        L.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE)
        L.ozgemm_free()
        del Ad, Bd, Cd, ws
        torch.cuda.empty_cache()
    return results


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--m", type=int, default=1024)
    p.add_argument("--n", type=int, default=1024)
    p.add_argument("--q", type=int, default=1024)
    p.add_argument("--s", type=str, default="8,9,10,11,12,13,14,15,16,17,18")
    p.add_argument("--phi", type=str, default="0.5")
    p.add_argument("--entries", type=int, default=1024)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--repeats", type=int, default=5)
    p.add_argument("--k", type=str, default="4,5,6,7,8", help="Scheme I slice counts")
    p.add_argument("--methods", type=str, default="ozaki2",
                   help="comma list of ozaki2, ozaki2-fast, ozaki2-accu, scheme1-rn, scheme1-hybrid")
    p.add_argument("--out", type=str, default="")
    a = p.parse_args(argv)
    res = run_sweep(a.m, a.n, a.q, _parse_list(a.s, int), _parse_list(a.phi, float), a.entries, a.seed, a.repeats,
                    _parse_list(a.k, int), _parse_list(a.methods, str))
    if a.out:
        with open(a.out, "w") as fh:
            json.dump(res, fh, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
