"""Host logic of bench.py, on the CPU: the refusal of more than one GPU, the
oracle baseline's worker pool (sizing, timing fields, bit-for-bit parity
accounting) on a tiny workload, and the lookup of the committed traffic
counters with its check of the product kernel's source hash."""
import importlib
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import ozaki2 as oz
from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    # imported by name, so that the spawned oracle workers can import it too
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    return importlib.import_module("bench")


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_cpu_baseline_pool_and_parity_accounting():
    """Two worker processes time the oracle on a block of a 96 x 40 x 96
    output; the 'GPU' result handed in is the oracle itself, so every entry
    must count as bit-exact, and a planted wrong entry must not."""
    bench = load_bench()
    m, q, n, s = 96, 40, 96, 12
    A, B = hpl_like(m, q, n, 1.0, seed=5)
    full = oz.dgemm(A, B, s)

    def getter(rows, cols):
        return full[np.ix_(rows, cols)]

    rec = bench.cpu_baseline(A, B, s, q, 1.0, getter, workers=2)
    assert rec["kind"] == "oracle" and rec["cores"] == 2 and rec["unit"] == "TFLOPS"
    assert rec["host_cpus"] >= 1 and rec["nproc"] >= 1
    entries = rec["parity_entries"]
    assert entries >= 8 * min(n, 256) and entries % min(n, 256) == 0
    assert rec["parity_bit_exact"] == entries
    assert rec["value"] == pytest.approx(2.0 * q * entries / rec["seconds"] / 1e12)
    assert rec["extrapolated_full_seconds"] == pytest.approx(rec["seconds"] * m * n / entries, rel=1e-3, abs=0.1)

    bad = full.copy()
    bad[7, 11] = np.nextafter(bad[7, 11], np.inf)

    def bad_getter(rows, cols):
        return bad[np.ix_(rows, cols)]

    rec2 = bench.cpu_baseline(A, B, s, q, 1.0, bad_getter, workers=2)
    rows_hit = rec2["parity_entries"] // min(n, 256)
    # row 7 is in the timed block only if the block covers it; the count
    # drops by exactly one when it does
    assert rec2["parity_bit_exact"] in (rec2["parity_entries"], rec2["parity_entries"] - 1)
    if rows_hit == m:
        assert rec2["parity_bit_exact"] == rec2["parity_entries"] - 1


def test_traffic_record_lookup():
    bench = load_bench()
    assert bench.traffic_record("no_such_workload") is None
    v = bench.traffic_record("ozaki2_dgemm_8192x8192x8192_s14_phi1")
    # the committed counters were taken on the current product kernel source
    assert isinstance(v, int) and v > 2 * 14 * 8192 * 8192
