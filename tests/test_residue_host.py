"""The residue arithmetic of the GPU kernels, run on the CPU.

``csrc/residue_arith.h`` (the code the residue kernels inline for every
entry and modulus) is compiled for the host with g++ and fed exact integers
A' held in doubles, in the three ranges its forms serve: |A'| < 2^50 (one
reduction), < 2^53 and < 2^78 (a split into 26-bit pieces, then one
reduction of a congruent integer below 2^35).  Every result must equal the
oracle's symmetric residue (``oracle.ozaki2.smod``, Ozaki II notes §6) for
all 20 greedy moduli: random magnitudes over the whole range, the range
ends, the piece boundaries 2^26 and 2^52 and their neighbours, and the
points where the quotient changes (r = -floor(m/2) and ceil(m/2) - 1).  A
wrong 2^52 constant, and the one-reduction form applied to wide A', must
both be caught.
"""
import math
import os
import random
import shutil
import struct
import subprocess

import numpy as np
import pytest

from oracle import ozaki2 as oz

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "residue_host_driver.cpp")
MODULI = oz.greedy_moduli(20)
LIMIT = {0: 2**50, 1: 2**53, 2: 2**78}


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("residue") / "residue_driver")
    subprocess.run([gxx, "-O2", "-std=c++17", "-ffp-contract=off", DRIVER, "-o", exe], check=True)
    return exe


def bits_hex(x: float) -> str:
    return format(struct.unpack("<Q", struct.pack("<d", x))[0], "x")


def run(driver, cases, plant=0):
    """cases: (form, m, A') with A' an exact integer held in a float."""
    text = "".join(f"{f} {m} {bits_hex(a)} {plant}\n" for f, m, a in cases)
    out = subprocess.run([driver], input=text, capture_output=True, text=True, timeout=300, check=True)
    return [int(v) for v in out.stdout.split()]


def representable(v: int) -> bool:
    return float(v) == v


def values(form: int, m: int, rng: random.Random):
    """Exact integers below LIMIT[form] in magnitude, each representable in
    a double."""
    lim = LIMIT[form]
    out = [0, 1, -1, m // 2, -(m // 2), (m + 1) // 2 - 1, -((m + 1) // 2), m, -m]
    # the largest integer-valued double below the limit
    top = float(lim - 1) if lim <= 2**53 else float(lim - 2 ** (lim.bit_length() - 1 - 53))
    out += [top, -top, float(lim // 2), -float(lim // 2)]
    for p in (26, 52):
        for d in (-1, 0, 1):
            v = 2**p + d
            if abs(v) < lim and representable(v):
                out += [v, -v]
        for k in (3, 255, 2**20 + 1):
            v = k * 2**p
            if abs(v) < lim and representable(v):
                out += [v, -v, v - 1 if representable(v - 1) else v]
    # around the points where floor(A'/m + 1/2) steps: A' = j m +- m/2
    for j in (1, 7, 2**30 + 3, 2**45 + 11):
        for off in (-((m + 1) // 2), (m + 1) // 2 - 1, -((m + 1) // 2) + 1, (m + 1) // 2):
            v = j * m + off
            if abs(v) < lim and representable(v):
                out += [v, -v]
    # random magnitudes across the range: a 53-bit significand at every scale
    for _ in range(120):
        e = rng.randrange(0, lim.bit_length() - 1)
        sig = rng.getrandbits(53) | (1 << 52)
        v = math.trunc(math.ldexp(sig, e - 52))
        if abs(v) >= lim:
            continue
        out.append(float(v) if rng.random() < 0.5 else -float(v))
    return [float(v) for v in out if abs(v) < lim]


@pytest.mark.parametrize("form", [0, 1, 2])
def test_residues_equal_the_oracle(driver, form):
    rng = random.Random(1000 + form)
    cases = []
    for m in MODULI:
        cases += [(form, m, a) for a in values(form, m, rng)]
    got = run(driver, cases)
    bad = []
    for (f, m, a), r in zip(cases, got):
        want = int(oz.smod(np.array([a]), m)[0])
        if r != want:
            bad.append((m, a, r, want))
    assert not bad, bad[:5]
    assert len(cases) > 20 * 150


def test_planted_mistakes_are_caught(driver):
    rng = random.Random(7)
    wide = [(2, m, a) for m in MODULI for a in values(2, m, rng) if abs(a) >= 2**52]
    for plant in (1, 2):
        got = run(driver, wide, plant=plant)
        wrong = sum(r != int(oz.smod(np.array([a]), m)[0]) for (_, m, a), r in zip(wide, got))
        assert wrong > len(wide) // 4, (plant, wrong, len(wide))
