"""The GEMM epilogue's reduction C''_t = C'_t mod m_t, run on the CPU.

``csrc/prod_mod.h`` (inlined by the GEMM kernel) is compiled for the host
with g++ and must agree with Python's floor-mod on int32 values: the whole
range's ends, every value next to a multiple of m at several magnitudes, and
exact multiples of m and their neighbours, and random values, for every modulus of the fixed list and a few others.
The biased form, which starts the accumulators at -(m-1)/2 and rounds to
nearest, is checked the same way for m = 256 and every odd m.
"""
import os
import random
import shutil
import subprocess

import pytest

from oracle import ozaki2 as oz

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "prod_mod_driver.cpp")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("pm") / "prod_mod_driver")
    subprocess.run([gxx, "-O2", "-std=c++17", "-ffp-contract=off", DRIVER, "-o", exe], check=True)
    return exe


def values(m: int, rng: random.Random) -> list[int]:
    lo, hi = -(2**31), 2**31 - 1
    vs = [lo, lo + 1, hi, hi - 1, 0, 1, -1, m, -m, m - 1, 1 - m]
    for mag in (m, 2**12, 2**20, 2**24, 2**28, 2**30, 2**31 - m):
        k = mag // m
        for base in (k * m, -k * m):
            vs += [base + d for d in (-1, 0, 1, m // 2, -(m // 2))]
    vs += [rng.randint(lo, hi) for _ in range(4000)]
    # exact multiples of m are where a floor without its half-step bias slips
    for _ in range(2000):
        base = rng.randint(lo // m, hi // m) * m
        vs += [base - 1, base, base + 1]
    return [v for v in vs if lo <= v <= hi]


def run_driver(driver, cases):
    text = "".join(f"{m} {len(vs)}\n" + "\n".join(map(str, vs)) + "\n" for m, vs in cases)
    out = subprocess.run([driver], input=text, capture_output=True, text=True, check=True).stdout.split()
    return iter(int(x) for x in out)


def test_mod_product_matches_floor_mod(driver):
    rng = random.Random(7)
    moduli = sorted(set(oz.greedy_moduli(20) + [2, 3, 7, 128, 129]))
    cases = [(m, values(m, rng)) for m in moduli]
    got = run_driver(driver, cases)
    for m, vs in cases:
        for v in vs:
            assert next(got) == v % m, (m, v)
            next(got)


def test_biased_mod_product_matches_floor_mod(driver):
    """The biased form (accumulator started at -(m-1)/2 for odd m, at 0 for
    m = 256) leaves v mod m in the low byte for every int32 accumulator;
    that holds for all odd m <= 255, so every odd m is checked."""
    rng = random.Random(11)
    moduli = sorted(set(oz.greedy_moduli(20) + list(range(3, 256, 2)) + [256]))
    cases = [(m, values(m, rng)[:600] + values(m, rng)[-600:]) for m in moduli]
    got = run_driver(driver, cases)
    checked = 0
    for m, vs in cases:
        h = 0 if m == 256 else (m - 1) // 2
        for v in vs:
            next(got)
            b = next(got)
            if v - h < -(2**31):
                assert b == -1
                continue
            assert b == v % m, (m, v)
            checked += 1
    assert checked > 0.99 * sum(len(vs) for _, vs in cases)
