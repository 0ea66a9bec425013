"""The block grid of the int8 product launches, run on the CPU.

``csrc/gemm_grid.h`` (used by the GEMM kernel and its host launcher) is
compiled with g++:

* ``tile_of_block`` must map the block ids of a launch one to one onto
  (plane, tile row, tile column), in both of its layouts (eighths of a plane
  per XCD, and whole planes per XCD for planes of at most 32 tiles), and in
  the whole-plane layout every block of a plane must sit on one XCD.
* ``choose_splits`` (K parts of a Scheme II product) must cover K with
  non-empty parts, keep every part exact in int32 once q_pad >= 2^17 (at most
  2^16 K entries: 2^16 * 2^14 < 2^31, the Ozaki II notes' block products),
  stay within its block cap, the workspace it is given and the region the
  configuration reserves, and keep the 16-bit sums of the reduction below
  2^16; on named shapes it must pick the expected counts.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "grid_driver.cpp")
SLICE = 128           # K entries per kernel slice
EXACT_SLICES = 512    # 2^16 K entries
BLOCK_CAP = 2048      # parts x moduli x tiles


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("grid") / "grid_driver")
    subprocess.run([gxx, "-O2", "-std=c++17", DRIVER, "-o", exe], check=True)
    return exe


def run(driver, text):
    return subprocess.run([driver], input=text, capture_output=True, text=True, check=True).stdout.split("\n")


MAP_CASES = [(np_, tm, tn) for np_ in (1, 3, 8, 14, 16, 24, 56, 112) for tm, tn in
             ((1, 1), (1, 3), (2, 2), (4, 4), (3, 5), (4, 8), (8, 4), (5, 7), (8, 8), (6, 11), (32, 32))]


def test_tile_map_is_a_bijection(driver):
    text = "".join(f"map {n} {tm} {tn}\n" for n, tm, tn in MAP_CASES)
    lines = iter(run(driver, text))
    for n, tm, tn in MAP_CASES:
        per = tm * tn
        seen = set()
        xcd_of_plane = {}
        for b in range(n * per):
            t, mi, nj = map(int, next(lines).split())
            assert 0 <= t < n and 0 <= mi < tm and 0 <= nj < tn, (n, tm, tn, b)
            seen.add((t, mi, nj))
            if per <= 32 and n % 8 == 0:
                assert xcd_of_plane.setdefault(t, b % 8) == b % 8, "a plane split over XCDs"
        assert len(seen) == n * per, (n, tm, tn)


def split_cases():
    cases = []
    for tiles in (1, 2, 4, 9, 16, 25, 32, 48, 64, 100, 256, 1024, 4096):
        for s in (1, 7, 8, 13, 14, 16, 20):
            for nk in (1, 2, 15, 31, 32, 33, 64, 100, 512, 1000, 1023, 1024, 1025, 1094, 4096, 8192, 2**20):
                for cap in (1, 10**9):
                    cases.append((tiles, s, nk, 256, cap))
    cases += [(16, 14, 512, cus, 10**9) for cus in (1, 32, 80, 304)]
    return cases


def test_split_choice_invariants(driver):
    cases = split_cases()
    text = "".join("split %d %d %d %d %d\n" % c for c in cases)
    lines = iter(run(driver, text))
    for tiles, s, nk, cus, cap in cases:
        parts, slices, region = map(int, next(lines).split())
        case = (tiles, s, nk, cus, cap, parts, slices)
        needs_blocks = nk >= 2 * EXACT_SLICES       # q_pad >= 2^17
        if parts == 0:                              # sequential K blocks
            assert needs_blocks, case
            continue
        assert parts >= 1 and slices >= 1, case
        assert parts * slices >= nk and (parts - 1) * slices < nk, case      # K covered, no empty part
        if needs_blocks:
            assert parts >= 2 and slices <= EXACT_SLICES, case               # each part exact in int32
        if parts > 1:
            assert parts <= 64, case                                         # 64 * 255 < 2^16
            assert parts * s * tiles <= BLOCK_CAP and parts * s <= cap, case
            assert parts * s * tiles * 256 * 256 <= region, case             # fits the reserved region
            assert slices >= 16 or needs_blocks, case
        else:
            assert slices == nk, case


@pytest.mark.parametrize("shape,want", [
    ((1024, 1024, 65536, 14), 8),     # skinny output, long K: 224 blocks -> 1792 = 7 waves
    ((2048, 2048, 65536, 14), 2),     # 896 blocks -> 1792
    ((8192, 8192, 8192, 14), 1),      # the square workload keeps one part
    ((16384, 16384, 1024, 14), 1),
    ((1024, 1024, 1024, 14), 1),      # too short to cut
    ((256, 256, 8192, 14), 4),
])
def test_split_choice_on_named_shapes(driver, shape, want):
    m, n, q, s = shape
    tiles = -(-m // 256) * -(-n // 256)
    nk = -(-q // SLICE)
    parts, _, _ = map(int, run(driver, f"split {tiles} {s} {nk} 256 {10**9}\n")[0].split())
    assert parts == want


def test_long_inner_dimension_uses_parts_when_they_fit(driver):
    # 512 x 2^20 x 512: 4 tiles, 8192 slices -> at least 16 parts of <= 2^16
    parts, slices, _ = map(int, run(driver, f"split 4 14 8192 256 {10**9}\n")[0].split())
    assert parts >= 16 and slices <= EXACT_SLICES
    # a large output with q >= 2^17 has no room for parts: sequential K blocks
    parts, _, _ = map(int, run(driver, f"split 1024 14 1025 256 {10**9}\n")[0].split())
    assert parts == 0
