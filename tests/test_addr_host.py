"""Every memory address of the product, residue and CRT kernels, emulated
on the CPU (tests/addr_driver.cpp): global loads and stores stay inside
their buffers and LDS accesses inside the block's allocation, for every
committed grid form at ragged and padded shapes.  No GPU is involved.

The driver restates the kernels' index arithmetic and uses the tile map and
K-part choice of csrc/gemm_grid.h itself.  A planted mistake -- the 32-byte
K slice with a row & 7 chunk swizzle that once overran the last residue
plane -- must be reported.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "addr_driver.cpp")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("addr") / "addr_driver")
    subprocess.run([gxx, "-O2", "-std=c++17", DRIVER, "-o", exe], check=True)
    return exe


def run(driver, lines):
    out = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    res = out.stdout.split("\n")[:-1]
    assert len(res) == sum(1 for l in lines if l.split()[0] in ("gemm", "plan", "reduce", "residue", "crt",
                                                                 "residue_pair", "scale_pair"))
    return res


def pad(x, r):
    return max(1, -(-x // r)) * r


def gemm_line(form, m, n, q, s, cus=256, parts=1, per=None, k_begin=0, k_slices=None, bug=0):
    mp, np_, qp = pad(m, 256), pad(n, 256), pad(q, 128)
    nk = qp // 128
    per = nk if per is None else per
    k_slices = per if k_slices is None else k_slices
    return f"gemm {form} {mp} {np_} {qp} {s} {cus} {parts} {per} {k_begin} {k_slices} {bug}"


SHAPES = [(1, 1, 1), (257, 255, 129), (300, 770, 1000), (513, 300, 4097)]


@pytest.mark.parametrize("m,n,q", SHAPES)
def test_product_forms_stay_in_bounds(driver, m, n, q):
    lines = [gemm_line("main", m, n, q, 3), gemm_line("ct", m, n, q, 2),
             # the persistent walk, with few compute units so that blocks take several tiles
             gemm_line("persist", m, n, q, 3, cus=5), gemm_line("persist", m, n, q, 14, cus=7),
             # eight wavefronts per block (blocks that walk few K slices)
             gemm_line("main8", m, n, q, 3), gemm_line("persist8", m, n, q, 14, cus=7)]
    for r in run(driver, lines):
        assert r.startswith("ok"), r


def test_k_parts_and_their_reduction(driver):
    # 256 x 256 x 8192 in 8 parts of 8 slices, and a ragged last part
    lines = [gemm_line("main", 256, 256, 8192, 14, parts=8, per=8),
             gemm_line("persist", 256, 256, 8192, 14, cus=9, parts=8, per=8),
             gemm_line("persist8", 256, 256, 8192, 14, cus=9, parts=8, per=8),
             gemm_line("main8", 200, 100, 8000, 3, parts=6, per=11),
             gemm_line("main", 200, 100, 8000, 3, parts=6, per=11),
             "reduce 256 256 14 8", "reduce 512 768 3 6"]
    for r in run(driver, lines):
        assert r.startswith("ok"), r


def test_sequential_k_blocks(driver):
    # q >= 2^17 without parts: launches of at most 512 slices, the later ones
    # adding to the residues already stored
    q = 2**17 + 300
    nk = pad(q, 128) // 128
    lines = [gemm_line("main", 300, 200, q, 2, k_begin=0, k_slices=512)]
    for k0 in range(512, nk, 512):
        lines.append(gemm_line("acc", 300, 200, q, 2, k_begin=k0, k_slices=min(512, nk - k0)))
    for r in run(driver, lines):
        assert r.startswith("ok"), r


def scheme1_plan(k, variant, r=32):
    """The plan entries of the Scheme I products, as the plan kernel builds them."""
    out = []
    if variant == "rn":
        for i in range(1, k + 1):
            for j in range(1, k - i + 2):
                out.append((i - 1, j - 1, 1, len(out)))
        return out
    for g in range(2, k + 2):
        s0 = 1
        while s0 <= g - 1:
            ln = min(r, g - s0)
            out.append((s0 - 1, g - s0 - 1, ln, len(out)))
            s0 += ln
    return sorted(out, key=lambda e: -e[2])


@pytest.mark.parametrize("plan,planes", [(scheme1_plan(4, "rn"), 4), (scheme1_plan(8, "hybrid", r=3), 8),
                                         ([(0, 0, 1, 0), (0, 1, 2, 1)], 2)])
def test_plan_form(driver, plan, planes):
    """Scheme I slice products and the two bound products of OS II-accu."""
    lines = [f"plan 512 256 1024 {planes} {planes} {len(plan)}"] + [" ".join(map(str, e)) for e in plan]
    for r in run(driver, lines):
        assert r.startswith("ok"), r


def test_crt_two_column_form_index_ranges(driver):
    """Outputs above 2^23 entries take two columns per thread (smaller ones
    one): a ragged 4100 x 2100 output, padded leading dimension."""
    for r in run(driver, [f"crt 4100 2100 {pad(4100, 256)} {pad(2100, 256)} 14 4103"]):
        assert r.startswith("ok"), r


@pytest.mark.parametrize("rows,q", [(1, 1), (300, 1000), (257, 129), (33, 4097)])
def test_residue_and_crt_index_ranges(driver, rows, q):
    rp, qp = pad(rows, 256), pad(q, 128)
    lines = [f"residue {rows} {rp} {q} {qp} 14 1 {rows + 3} 0",   # A: rows contiguous, lda = rows + 3
             f"residue {rows} {rp} {q} {qp} 14 {q + 1} 1 0",      # B: the inner dimension contiguous
             f"crt {rows} {rows // 2 + 1} {rp} {pad(rows // 2 + 1, 256)} 14 {rows + 5}",
             f"crt {rows} 3 {rp} 256 20 {rows}"]
    if 4096 <= q <= 8192:
        lines.append(f"residue {rows} {rp} {q} {qp} 14 {q} 1 1")  # B in one pass
    for r in run(driver, lines):
        assert r.startswith("ok"), r


@pytest.mark.parametrize("m,n,q", [(1, 1, 1), (300, 257, 1000), (257, 33, 129), (1024, 1024, 1024)])
def test_pair_launches_stay_in_bounds(driver, m, n, q):
    """The one-launch forms of A's and B's residue passes and of their scale
    passes: every block decodes to a tile of the two separate grids, each
    tile comes up once, and every access stays inside its buffer; with the
    row-exponent finalisation folded in, every row's exponent is stored
    exactly once."""
    mp, np_, qp = pad(m, 256), pad(n, 256), pad(q, 128)
    lines = [f"residue_pair {m} {mp} {m + 3} {n} {np_} {q + 1} {q} {qp} 14 0 0",
             f"residue_pair {m} {mp} {m} {n} {np_} {q} {q} {qp} 20 0 0"]
    for nch in (1, 8, min(128, max(1, q // 8))):
        lines.append(f"scale_pair {m} {mp} {m + 5} {n} {q + 2} {q} {nch}")
        # the row-exponent finalisation folded into the residue pass: the
        # partial maxima the scale pass wrote (stride m_pad, or a larger
        # configured one), and one exponent store per row
        lines.append(f"residue_pair {m} {mp} {m + 3} {n} {np_} {q + 1} {q} {qp} 14 {mp} {nch}")
        lines.append(f"residue_pair {m} {mp} {m} {n} {np_} {q} {q} {qp} 14 {mp + 512} {nch}")
    for r in run(driver, lines):
        assert r.startswith("ok"), r


def test_planted_swizzle_overrun_is_caught(driver):
    """32-byte K slices with the row & 7 swizzle address chunks 0..7 of a
    two-chunk row: the emulation reports the access outside the buffer (on
    the four-wavefront int32 form with 32 x 32 tiles that the faulting
    probe used; the same form without the planted slice is in bounds)."""
    res = run(driver, [gemm_line("ct4", 256, 256, 256, 2, bug=1), gemm_line("ct4", 256, 256, 256, 2)])
    assert res[0].startswith("bad") and res[1].startswith("ok")
