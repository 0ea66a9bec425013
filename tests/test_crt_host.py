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


def limbs(v: int, n: int, width: int):
    return [(v >> (width * i)) & ((1 << width) - 1) for i in range(n)]


def width_for(M: int) -> int:
    """Limb width the library uses: 40 bits while three limbs hold M."""
    return 40 if M.bit_length() <= 120 else 32


def run_cases(exe, s, cases, width=None):
    mods = oz.greedy_moduli(s)
    M, Mt, yt = oz.crt_constants(mods)
    W = [a * b for a, b in zip(Mt, yt)]
    w = width or width_for(M)
    L = (M.bit_length() + w - 1) // w
    lines = [" ".join(str(v) for v in [w, L] + limbs(M, 5, w) + limbs(M // 2, 5, w)),
             f"{bits(float(M // 2)):016x} {bits(1.0 / float(M)):016x}", str(len(cases))]
    for X, scale in cases:
        r = [X % m for m in mods]
        S = [sum(rt * ((Wt >> (w * l)) & ((1 << w) - 1)) for rt, Wt in zip(r, W)) for l in range(L)]
        assert all(0 <= v < 2**53 for v in S)
        lines.append(" ".join(str(v) for v in [scale] + S))
    out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
    got = [int(x, 16) for x in out.stdout.split()]
    assert len(got) == len(cases)
    return got, M


def expected(X, scale):
    return bits(oz.round_scaled(X, scale))


CASES_S = [1, 2, 3, 4, 5, 8, 9, 13, 14, 15, 16, 18, 20]


@pytest.mark.parametrize("width", [32, 40])
@pytest.mark.parametrize("s", CASES_S)
def test_random_and_boundary(driver, s, width):
    M0, _, _ = oz.crt_constants(oz.greedy_moduli(s))
    if width == 40 and M0.bit_length() > 120:
        pytest.skip("40-bit limbs are used while three of them hold M")
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
    got, _ = run_cases(driver, s, cases, width)
    for (X, scale), g in zip(cases, got):
        assert g == expected(X, scale), (s, width, X, scale, hex(g), hex(expected(X, scale)))


@pytest.mark.parametrize("width", [32, 40])
def test_ties_round_to_even(driver, width):
    s = 14
    M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
    cases = []
    # a tie (or one unit off it) at the 53-bit position for leading bits in
    # every limb, so that the deciding bits sit in lower limbs
    for top in (54, 60, 79, 80, 85, 100, 108):
        for lowbits in (1, 3, 5):
            base = (1 << top) + (lowbits << (top - 53))
            for X in (base, base + 1, base - 1, base + (1 << 39), base - (1 << 41)):
                cases += [(X, -50), (-X, 0)]
    got, _ = run_cases(driver, s, cases, width)
    for (X, scale), g in zip(cases, got):
        assert g == expected(X, scale), (X, scale)


@pytest.mark.parametrize("width", [32, 40])
def test_subnormal_results_round_once(driver, width):
    """X with more than 53 significant bits whose scaled value is subnormal
    and sits on, or one unit beside, a tie of the subnormal grid: rounding
    X to 53 bits first and then to the grid would go wrong here."""
    s = 14
    M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
    cases = []
    for top in (60, 80, 100, 108):
        for keep in (1, 2, 10, 30, 52):
            scale = keep - 1 - 1074 - top  # leading bit of X 2^scale at 2^(keep - 1075)
            for odd in (1, 3):
                tie = (1 << top) + odd * (1 << (top - keep))
                for X in (tie - 1, tie, tie + 1):
                    if 2 * X < M:
                        cases += [(X, scale), (-X, scale)]
    got, _ = run_cases(driver, s, cases, width)
    for (X, scale), g in zip(cases, got):
        assert g == expected(X, scale), (width, X, scale, hex(g), hex(expected(X, scale)))
