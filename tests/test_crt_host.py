"""The CRT reconstruction arithmetic of the GPU kernel, run on the CPU.

``csrc/crt_reconstruct.h`` (the code the CRT kernel inlines) is compiled for
the host with g++ and fed limb sums S_l = sum_t r_t w_{t,l} for chosen
integers X.  Its result must equal the oracle's single rounding of the
symmetric representative times 2^scale, bit for bit.  Cases cover random X,
X next to +-M/2 (the exact-comparison band), tiny X, X = 0, and scales that
land in the subnormal range, on rounding ties and past the double range.
"""
import math
import os
import random
import shutil
import struct
import subprocess

import pytest

from oracle import ozaki2 as oz

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "crt_host_driver.cpp")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("crt") / "crt_driver")
    subprocess.run([gxx, "-O2", "-std=c++17", "-ffp-contract=off", DRIVER, "-o", exe], check=True)
    return exe


def bits(x: float) -> int:
    return struct.unpack("<Q", struct.pack("<d", x))[0]


def limbs32(v: int, n: int):
    return [(v >> (32 * i)) & 0xFFFFFFFF for i in range(n)]


def run_cases(exe, s, cases):
    mods = oz.greedy_moduli(s)
    M, Mt, yt = oz.crt_constants(mods)
    W = [a * b for a, b in zip(Mt, yt)]
    L = (M.bit_length() + 31) // 32
    lines = [" ".join(str(v) for v in [L] + limbs32(M, 5) + limbs32(M // 2, 5)),
             f"{bits(float(M // 2)):016x} {bits(1.0 / float(M)):016x}", str(len(cases))]
    for X, scale in cases:
        r = [X % m for m in mods]
        S = [sum(rt * ((Wt >> (32 * l)) & 0xFFFFFFFF) for rt, Wt in zip(r, W)) for l in range(L)]
        assert all(0 <= v < 2**46 for v in S)
        lines.append(" ".join(str(v) for v in [scale] + S))
    out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
    got = [int(x, 16) for x in out.stdout.split()]
    assert len(got) == len(cases)
    return got, M


def expected(X, scale):
    return bits(oz.round_scaled(X, scale))


@pytest.mark.parametrize("s", [1, 2, 3, 4, 5, 8, 9, 13, 14, 16, 18, 20])
def test_random_and_boundary(driver, s):
    rng = random.Random(100 + s)
    M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
    half = M // 2
    cases = []
    for _ in range(300):
        X = rng.randrange(-half + 1, half)
        cases.append((X, rng.randrange(-1200, 200)))
    for d in list(range(1, 40)) + [2**20, 2**40 + 3]:  # next to +-M/2, inside the range
        if d < half:
            cases += [(half - d, -100), (-(half - d), -100)]
    cases += [(0, 0), (1, 0), (-1, 0), (1, -1074), (1, -1075), (3, -1075), (-3, -1076), (5, -1076)]
    big = (1 << 53) + 1
    if big < half:
        cases += [(big, 0), (-big, 3), (big + 2, -1100)]
    top = half - 1
    cases += [(top, 1024 - top.bit_length()), (-top, 1023 - top.bit_length() + 1)]
    got, _ = run_cases(driver, s, cases)
    for (X, scale), g in zip(cases, got):
        assert g == expected(X, scale), (s, X, scale, hex(g), hex(expected(X, scale)))


def test_ties_round_to_even(driver):
    s = 14
    M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
    cases = []
    for base in [(1 << 60) + (1 << 7), (1 << 60) + (3 << 7), (1 << 100) + (1 << 47), (1 << 100) + (3 << 47)]:
        cases += [(base, -50), (-base, -50), (base + 1, 0), (base - 1, 0)]
    got, _ = run_cases(driver, s, cases)
    for (X, scale), g in zip(cases, got):
        assert g == expected(X, scale), (X, scale)
