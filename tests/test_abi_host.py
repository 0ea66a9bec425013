"""Host-side checks of the C-ABI library (no GPU needed).

The library must load and export every function ``include/ozgemm.h``
declares; the host-only entry points (moduli, bit budget, workspace and
plane sizes, argument validation) must agree with the oracle and the header.
No call here reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

from oracle import ozaki2 as oz
from fp64_gemm_emulation_ozii_amd import ozgemm as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ozgemm.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libozgemm.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ozgemm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_what_binding_lists():
    assert declared_functions() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


@pytest.mark.parametrize("s", range(1, 21))
def test_moduli_match_oracle(s):
    assert L.ozgemm_moduli(s) == oz.greedy_moduli(s)


def test_moduli_rejects_bad_s():
    with pytest.raises(L.OzgemmError):
        L.ozgemm_moduli(0)
    with pytest.raises(L.OzgemmError):
        L.ozgemm_moduli(21)


@pytest.mark.parametrize("q", [1, 2, 3, 63, 64, 65, 127, 1000, 1024, 4096, 8192, 16384, 65536, 2**17 - 1])
def test_kbits_match_oracle(q):
    for s in range(1, 21):
        M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
        want = oz.kbits(M, q)
        got = L.ozgemm_kbits(s, q)
        if want < 0:
            assert got < 0
        else:
            assert got == want, (s, q)


def test_kbits_accepts_long_k_and_rejects_q_max():
    assert L.ozgemm_kbits(14, 2**17) == oz.kbits(oz.crt_constants(oz.greedy_moduli(14))[0], 2**17)
    assert L.ozgemm_kbits(14, 2**20) == oz.kbits(oz.crt_constants(oz.greedy_moduli(14))[0], 2**20)
    assert L.ozgemm_kbits(14, L.OZGEMM_Q_MAX + 1) < 0


def test_workspace_and_plane_dims():
    mp, np_, qp = L.ozgemm_plane_dims(300, 257, 1000)
    assert mp % 256 == 0 and mp >= 300 and np_ % 256 == 0 and np_ >= 257 and qp % 128 == 0 and qp >= 1000
    small = L.ozgemm_workspace_bytes(64, 64, 64, 14)
    big = L.ozgemm_workspace_bytes(8192, 8192, 8192, 14)
    assert 0 < small < big
    # the residue planes alone: s (m_pad + n_pad) q_pad, plus s m_pad n_pad product residues
    assert big >= 14 * (8192 + 8192) * 8192 + 14 * 8192 * 8192
    assert L.ozgemm_workspace_bytes(64, 64, 64, 0) == 0
    assert L.ozgemm_workspace_bytes(64, 64, 64, 21) == 0


def test_strerror_texts():
    assert "argument 3" in L.ozgemm_strerror(-3)
    assert "config" in L.ozgemm_strerror(L.OZGEMM_NOT_CONFIGURED)
    assert "2^27" in L.ozgemm_strerror(L.OZGEMM_RANGE) and "2^23" in L.ozgemm_strerror(L.OZGEMM_RANGE)


FAKE = 1 << 40  # a non-NULL address that no validation path dereferences


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# Every call below must return from argument validation.  As a guard against a
# regression that would let one reach a kernel launch with these fake
# addresses, the validation tests only run where no GPU is visible.
no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer validation runs only without a GPU")


@no_gpu_only
def test_validation_before_any_launch():
    lib = L.lib()
    lib.ozgemm_free()
    assert lib.ozgemm_dgemm(8, 8, 8, FAKE, 8, FAKE, 8, FAKE + (1 << 30), 8, 14) == L.OZGEMM_NOT_CONFIGURED
    ws = L.ozgemm_workspace_bytes(512, 512, 512, 16)
    assert lib.ozgemm_config(16, 512, 512, 512, None, FAKE, ws - 1) == L.OZGEMM_WORKSPACE_TOO_SMALL
    assert lib.ozgemm_config(0, 512, 512, 512, None, FAKE, ws) == -1
    assert lib.ozgemm_config(16, -1, 512, 512, None, FAKE, ws) == -2
    assert lib.ozgemm_config(16, 512, 512, L.OZGEMM_Q_MAX + 1, None, FAKE, ws) == -4
    # rows padded to 256 must form at most 65535 tiles of 32 (the residue grid's y)
    assert L.OZGEMM_MAX_ROWS == 2**21 - 256 and -(-L.OZGEMM_MAX_ROWS // 256) * 256 // 32 <= 65535
    assert -(-(L.OZGEMM_MAX_ROWS + 1) // 256) * 256 // 32 > 65535
    big = L.ozgemm_workspace_bytes(L.OZGEMM_MAX_ROWS, 1, 1, 1)
    assert lib.ozgemm_config(1, L.OZGEMM_MAX_ROWS, 1, 1, None, FAKE, big) == 0
    assert lib.ozgemm_config(1, L.OZGEMM_MAX_ROWS + 1, 1, 1, None, FAKE, big) == -2
    big = L.ozgemm_workspace_bytes(1, L.OZGEMM_MAX_ROWS, 1, 1)
    assert lib.ozgemm_config(1, 1, L.OZGEMM_MAX_ROWS, 1, None, FAKE, big) == 0
    assert lib.ozgemm_config(1, 1, L.OZGEMM_MAX_ROWS + 1, 1, None, FAKE, big) == -3
    assert lib.ozgemm_config(16, 512, 512, 512, None, None, ws) == -6
    assert lib.ozgemm_config(16, 512, 512, 512, None, FAKE, ws) == 0
    Cp = FAKE + (1 << 30)
    d = lib.ozgemm_dgemm
    assert d(-1, 8, 8, FAKE, 8, FAKE, 8, Cp, 8, 14) == -1
    assert d(8, -1, 8, FAKE, 8, FAKE, 8, Cp, 8, 14) == -2
    assert d(8, 8, -1, FAKE, 8, FAKE, 8, Cp, 8, 14) == -3
    assert d(8, 8, 8, None, 8, FAKE, 8, Cp, 8, 14) == -4
    assert d(8, 8, 8, FAKE, 7, FAKE, 8, Cp, 8, 14) == -5
    assert d(8, 8, 8, FAKE, 8, None, 8, Cp, 8, 14) == -6
    assert d(8, 8, 8, FAKE, 8, FAKE, 7, Cp, 8, 14) == -7
    assert d(8, 8, 8, FAKE, 8, FAKE, 8, None, 8, 14) == -8
    assert d(8, 8, 8, FAKE, 8, FAKE, 8, Cp, 7, 14) == -9
    assert d(8, 8, 8, FAKE, 8, FAKE, 8, Cp, 8, 0) == -10
    assert d(8, 8, 8, FAKE, 8, FAKE, 8, Cp, 8, 21) == -10
    assert d(8, 8, 8, FAKE, 8, FAKE, 8, Cp, 8, 17) == L.OZGEMM_RANGE        # s above s_max
    assert d(513, 8, 8, FAKE, 513, FAKE, 8, Cp, 513, 14) == L.OZGEMM_RANGE  # m above max_m
    assert d(8, 8, 600, FAKE, 8, FAKE, 600, Cp, 8, 14) == L.OZGEMM_RANGE    # q above max_q
    assert d(8, 8, 64, FAKE, 8, FAKE, 64, Cp, 8, 1) == L.OZGEMM_RANGE       # s = 1 leaves k < 1
    # C overlapping A
    assert d(8, 8, 8, FAKE, 8, FAKE + (1 << 20), 8, FAKE + 64, 8, 14) == -8
    # empty problems return before touching memory
    assert d(0, 8, 8, FAKE, 1, FAKE, 8, Cp, 1, 14) == 0
    assert d(8, 0, 8, FAKE, 8, FAKE, 8, Cp, 8, 14) == 0
    lib.ozgemm_free()


@no_gpu_only
def test_config_rejects_q_limit_and_stage_checks():
    lib = L.lib()
    ws = L.ozgemm_workspace_bytes(256, 256, 256, 14)
    assert lib.ozgemm_config(14, 256, 256, 256, None, FAKE, ws) == 0
    assert lib.ozgemm_stage_gemm(8, 8, 0, 14, FAKE, FAKE, None, None) == -3
    assert lib.ozgemm_stage_gemm(8, 8, 8, 15, FAKE, FAKE, None, None) == L.OZGEMM_RANGE
    assert lib.ozgemm_stage_crt(8, 8, 8, 14, None, FAKE, FAKE, FAKE, 8) == -5
    assert lib.ozgemm_stage_residue(8, 8, 8, 14, FAKE, 8, FAKE, 8, FAKE, FAKE, None, FAKE, None, None) == -11
    lib.ozgemm_free()


# ------------------------------------------------------------ Scheme I host side

from oracle import ozaki1 as o1  # noqa: E402


@pytest.mark.parametrize("q", [1, 2, 3, 64, 1000, 4096, 4097, 65536, 2**17 + 3, 2**20, 2**23, 2**29, 2**29 + 1])
def test_scheme1_beta_matches_oracle(q):
    try:
        ref = o1.slice_width(q)
    except ValueError:
        ref = -1
    assert L.ozgemm_scheme1_beta(q) == ref


@pytest.mark.parametrize("q", [64, 4096, 65536, 2**20])
@pytest.mark.parametrize("k", [1, 2, 4, 8, 16])
def test_scheme1_outputs_match_oracle(q, k):
    beta = o1.slice_width(q)
    r = o1.group_size(q, beta)
    assert L.ozgemm_scheme1_outputs(k, L.OZGEMM_S1_RN, q) == len(o1.triangle(k))
    assert L.ozgemm_scheme1_outputs(k, L.OZGEMM_S1_HYBRID, q) == len(o1.groups(k, r))


def test_scheme1_host_validation():
    assert L.ozgemm_scheme1_outputs(0, 0, 64) < 0
    assert L.ozgemm_scheme1_outputs(17, 0, 64) < 0
    assert L.ozgemm_scheme1_outputs(4, 2, 64) < 0
    assert L.ozgemm_scheme1_workspace_bytes(64, 64, 64, 0, 0) == 0
    assert L.ozgemm_scheme1_workspace_bytes(64, 64, 64, 4, 5) == 0
    w = L.ozgemm_scheme1_workspace_bytes(1000, 700, 300, 8, L.OZGEMM_S1_RN)
    mp, np_, qp = L.ozgemm_plane_dims(1000, 700, 300)
    # at least the slices and the 36 int32 product planes
    assert w >= 8 * (mp + np_) * qp + 36 * mp * np_ * 4
    assert L.ozgemm_scheme1_workspace_bytes(1000, 700, 300, 8, L.OZGEMM_S1_HYBRID) < w


@no_gpu_only
def test_scheme1_validation_before_any_launch():
    lib = L.lib()
    lib.ozgemm_free()
    Cp = FAKE + (1 << 30)
    d = lib.ozgemm_scheme1_dgemm
    assert d(8, 8, 8, FAKE, 8, FAKE, 8, Cp, 8, 4, 0) == L.OZGEMM_NOT_CONFIGURED
    ws = L.ozgemm_workspace_bytes(256, 256, 256, 14)
    assert lib.ozgemm_config(14, 256, 256, 256, None, FAKE, ws) == 0
    assert d(-1, 8, 8, FAKE, 8, FAKE, 8, Cp, 8, 4, 0) == -1
    assert d(8, 8, 8, FAKE, 7, FAKE, 8, Cp, 8, 4, 0) == -5
    assert d(8, 8, 8, FAKE, 8, FAKE, 8, None, 8, 4, 0) == -8
    assert d(8, 8, 8, FAKE, 8, FAKE, 8, Cp, 7, 4, 0) == -9
    assert d(8, 8, 8, FAKE, 8, FAKE, 8, Cp, 8, 0, 0) == -10
    assert d(8, 8, 8, FAKE, 8, FAKE, 8, Cp, 8, 17, 0) == -10
    assert d(8, 8, 8, FAKE, 8, FAKE, 8, Cp, 8, 4, 2) == -11
    assert d(8, 8, 2**29 + 1, FAKE, 8, FAKE, 2**29 + 1, Cp, 8, 4, 0) == L.OZGEMM_RANGE
    # a Scheme II sized workspace is too small for a larger Scheme I problem
    assert d(2048, 2048, 2048, FAKE, 2048, FAKE, 2048, FAKE + (1 << 36), 2048, 8, 0) == L.OZGEMM_WORKSPACE_TOO_SMALL
    assert d(0, 8, 8, FAKE, 1, FAKE, 8, Cp, 1, 4, 0) == 0
    s = lib.ozgemm_scheme1_stage_split
    assert s(8, 8, 8, 4, 0, FAKE, 8, FAKE, 8, None, FAKE, FAKE, FAKE) == -10
    assert s(8, 8, 8, 4, 3, FAKE, 8, FAKE, 8, FAKE, FAKE, FAKE, FAKE) == -9
    p = lib.ozgemm_scheme1_stage_products
    assert p(8, 8, 8, 4, 0, FAKE, FAKE, None) == -8
    a = lib.ozgemm_scheme1_stage_accumulate
    assert a(8, 8, 8, 4, 0, FAKE, FAKE, FAKE, FAKE, 7) == -10
    lib.ozgemm_free()


def test_binding_constants_match_the_header():
    """Every integer #define of include/ozgemm.h that the binding mirrors has
    the same value there."""
    import os
    import re
    here = os.path.dirname(os.path.abspath(__file__))
    text = open(os.path.join(here, "..", "include", "ozgemm.h")).read()
    seen = 0
    for name, expr in re.findall(r"^#define\s+(OZGEMM_\w+)\s+([^/\n]+)", text, flags=re.M):
        if not hasattr(L, name):
            continue
        value = eval(expr.strip(), {})  # integer literals and shifts only
        assert getattr(L, name) == value, name
        seen += 1
    assert seen >= 10


def test_fast_budget_rejects_q_beyond_exact_norm_sums():
    """OS II-fast sums q squared terms of at most 2^40 into 64 bits; the
    library refuses q >= 2^23, the oracle's own limit (row_norm_units)."""
    lim = L.OZGEMM_FAST_Q_LIMIT
    assert lim == 2**23
    a, b = L.ozgemm_bound_budget(14, lim - 1, L.OZGEMM_BOUND_FAST)
    assert (a, b) == oz.cs_budget(oz.crt_constants(oz.greedy_moduli(14))[0])
    st = L.lib().ozgemm_bound_budget(14, lim, L.OZGEMM_BOUND_FAST, ctypes.byref(ctypes.c_int()),
                                     ctypes.byref(ctypes.c_int()))
    assert st == L.OZGEMM_RANGE
    # the conservative budget has no such limit
    assert L.ozgemm_bound_budget(14, lim, L.OZGEMM_BOUND_CONSERVATIVE)[0] == L.ozgemm_kbits(14, lim)


@no_gpu_only
def test_fast_budget_q_limit_before_any_launch():
    lib = L.lib()
    lim = L.OZGEMM_FAST_Q_LIMIT
    ws = L.ozgemm_workspace_bytes(8, 8, lim, 14)
    assert lib.ozgemm_config(14, 8, 8, lim, None, FAKE, ws) == 0
    Cp = FAKE + (1 << 40)
    assert lib.ozgemm_set_bound(L.OZGEMM_BOUND_FAST) == 0
    e = ctypes.c_void_p(FAKE + (1 << 41))
    assert lib.ozgemm_dgemm(8, 8, lim, FAKE, 8, FAKE, lim, Cp, 8, 14) == L.OZGEMM_RANGE
    assert lib.ozgemm_stage_scale(8, 8, lim, 14, FAKE, 8, FAKE, lim, e, e) == L.OZGEMM_RANGE
    assert lib.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE) == 0
    lib.ozgemm_free()


@pytest.mark.parametrize("s", [2, 8, 14, 20])
def test_accu_budget_matches_oracle(s):
    M = oz.crt_constants(oz.greedy_moduli(s))[0]
    if oz.kbits(M, 500) < 1:
        assert L.lib().ozgemm_bound_budget(s, 500, L.OZGEMM_BOUND_ACCU, ctypes.byref(ctypes.c_int()),
                                           ctypes.byref(ctypes.c_int())) == L.OZGEMM_RANGE
        return
    assert L.ozgemm_bound_budget(s, 500, L.OZGEMM_BOUND_ACCU) == ((M // 2 - 1).bit_length() - 1, oz.ACCU_KMAX)


def test_accu_mode_constants_and_limits():
    assert L.OZGEMM_ACCU_Q_MAX == 2**16
    # the bound products stay exact in int32 up to that length
    assert 2 * oz.ACCU_RES**2 * L.OZGEMM_ACCU_Q_MAX < 2**31
    lib = L.lib()
    out = (ctypes.byref(ctypes.c_int()), ctypes.byref(ctypes.c_int()))
    assert lib.ozgemm_bound_budget(14, 2**16 + 1, L.OZGEMM_BOUND_ACCU, *out) == L.OZGEMM_RANGE
    assert lib.ozgemm_bound_budget(14, 500, 3, *out) == -3
    assert lib.ozgemm_set_bound(3) == -1
    assert lib.ozgemm_set_bound(L.OZGEMM_BOUND_ACCU) == 0
    assert lib.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE) == 0


@no_gpu_only
def test_accu_checks_before_any_launch():
    lib = L.lib()
    ws = L.ozgemm_workspace_bytes(8, 8, 2**17, 14)
    assert lib.ozgemm_config(14, 8, 8, 2**17, None, FAKE, ws) == 0
    Cp = FAKE + (1 << 40)
    assert lib.ozgemm_set_bound(L.OZGEMM_BOUND_ACCU) == 0
    e = ctypes.c_void_p(FAKE + (1 << 41))
    q = L.OZGEMM_ACCU_Q_MAX + 1
    assert lib.ozgemm_dgemm(8, 8, q, FAKE, 8, FAKE, q, Cp, 8, 14) == L.OZGEMM_RANGE
    assert lib.ozgemm_stage_scale(8, 8, q, 14, FAKE, 8, FAKE, q, e, e) == L.OZGEMM_RANGE
    # s_max = 2 and a 1024 x 1024 output: no room for the bound's planes
    ws = L.ozgemm_workspace_bytes(1024, 1024, 64, 2)
    assert lib.ozgemm_config(2, 1024, 1024, 64, None, FAKE, ws) == 0
    assert lib.ozgemm_set_bound(L.OZGEMM_BOUND_ACCU) == 0
    assert lib.ozgemm_dgemm(1024, 1024, 64, FAKE, 1024, FAKE, 64, Cp, 1024, 2) == L.OZGEMM_WORKSPACE_TOO_SMALL
    assert lib.ozgemm_stage_scale(1024, 1024, 64, 2, FAKE, 1024, FAKE, 64, e, e) == L.OZGEMM_WORKSPACE_TOO_SMALL
    assert lib.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE) == 0
    lib.ozgemm_free()


def test_mfma_ceiling_argument_checks():
    """The matrix-core rate probe rejects bad arguments before any launch."""
    lib = L.lib()
    sink = ctypes.c_void_p(FAKE)
    assert lib.ozgemm_mfma_ceiling(0, 4, 1, sink, None) == -1
    assert lib.ozgemm_mfma_ceiling((1 << 20) + 1, 4, 1, sink, None) == -1
    assert lib.ozgemm_mfma_ceiling(4, 0, 1, sink, None) == -2
    assert lib.ozgemm_mfma_ceiling(4, 4, 1, None, None) == -4
