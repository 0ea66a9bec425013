"""The exact budget comparison of OS II-accu as the combine kernel evaluates
it (csrc/accu_budget.h, built for the host with g++): floor(log2(V / N)) from
the top 64 bits of V = (M/2 - 1) 127^2 2^14 and its bit length, against
Python integers, for every s and for N at powers of two, next to the
decision points V / 2^t and at random.  No GPU is involved."""
import os
import random
import shutil
import subprocess

import pytest

from oracle import ozaki2 as oz

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "accu_budget_driver.cpp")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("accu") / "accu_budget_driver")
    subprocess.run([gxx, "-O2", "-std=c++17", DRIVER, "-o", exe], check=True)
    return exe


def cases_for(V: int, rng: random.Random):
    out = set()
    for b in range(0, 62):
        out.add(1 << b)
        out.add((1 << (b + 1)) - 1)
    for t in range(V.bit_length() - 62, V.bit_length()):
        d = V >> t  # N <= d  <=>  N 2^t <= V
        for n in (d - 1, d, d + 1):
            if 0 < n < 2**62:
                out.add(n)
    for _ in range(300):
        out.add(rng.randrange(1, 2**62))
    return sorted(out)


def test_floor_log2_ratio_matches_python_integers(driver):
    rng = random.Random(12)
    lines, expect = [], []
    for s in range(1, 21):
        M = oz.crt_constants(oz.greedy_moduli(s))[0]
        V = (M // 2 - 1) * oz.ACCU_DEN
        if V.bit_length() < 64:
            continue  # the library needs s >= 2; such small V never reaches the kernel
        bv = V.bit_length()
        vtop = V >> (bv - 64)
        ns = cases_for(V, rng)
        lines.append(f"{vtop} {bv} {len(ns)}")
        lines.extend(str(n) for n in ns)
        expect.extend((V // n).bit_length() - 1 for n in ns)
    res = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
    got = [int(x) for x in res.stdout.split()]
    assert got == expect

