"""ctypes binding of ``libozgemm.so`` (the C-ABI declared in ``include/ozgemm.h``).

Functions carry the C names and only marshal arguments: torch tensors become
device pointers, ``None`` becomes NULL, the stream defaults to torch's
current stream.  Every step of the computation runs in the HIP library; if
the library is missing this module raises instead of computing anything.

A non-zero status raises :class:`OzgemmError` (with ``ozgemm_strerror``'s
text) unless the function is documented to return a value.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libozgemm.so")

OZGEMM_OK = 0
OZGEMM_NOT_CONFIGURED = 1
OZGEMM_RANGE = 2
OZGEMM_WORKSPACE_TOO_SMALL = 3
OZGEMM_HIP_ERROR = 4
OZGEMM_S_MAX = 20
OZGEMM_PANELS_MAX = 16
OZGEMM_Q_LIMIT = 1 << 17
OZGEMM_Q_MAX = 1 << 27
OZGEMM_FAST_Q_LIMIT = 1 << 23  # OS II-fast needs q below this
OZGEMM_NOALLOC_BYTES = 128 << 20  # the fixed device array of ozgemm_dgemm_noalloc
OZGEMM_MAX_ROWS = 2096896  # 2^21 - 256
OZGEMM_ONE_PASS_Q_MIN = 4096  # B read once by ozgemm_dgemm for q in [MIN, MAX] (conservative budget)
OZGEMM_ONE_PASS_Q_MAX = 8192
OZGEMM_EXP_NONFINITE = 0x7FFFFFFF
OZGEMM_BOUND_CONSERVATIVE = 0
OZGEMM_BOUND_FAST = 1
OZGEMM_BOUND_ACCU = 2
OZGEMM_ACCU_Q_MAX = 1 << 16
OZGEMM_S1_RN = 0
OZGEMM_S1_HYBRID = 1
OZGEMM_S1_K_MAX = 16
OZGEMM_S1_MAX_OUT = 136

#: every symbol the header declares
EXPORTS = (
    "ozgemm_workspace_bytes", "ozgemm_config", "ozgemm_set_stream", "ozgemm_free", "ozgemm_strerror",
    "ozgemm_dgemm", "ozgemm_moduli", "ozgemm_kbits", "ozgemm_plane_dims", "ozgemm_stage_scale",
    "ozgemm_stage_residue", "ozgemm_stage_gemm", "ozgemm_stage_crt", "ozgemm_timing", "ozgemm_phase_ms",
    "ozgemm_scheme1_beta", "ozgemm_scheme1_outputs", "ozgemm_scheme1_workspace_bytes", "ozgemm_scheme1_dgemm",
    "ozgemm_scheme1_stage_split", "ozgemm_scheme1_stage_products", "ozgemm_scheme1_stage_accumulate",
    "ozgemm_set_bound", "ozgemm_bound_budget", "ozgemm_gemm_parts", "ozgemm_phase_calls",
    "ozgemm_dgemm_noalloc", "ozgemm_set_panels", "ozgemm_mfma_ceiling",
)

_lib = None
_workspace = None  # keeps a library-config workspace tensor alive


class OzgemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {ozgemm_strerror(status)}")


def lib():
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fp64_gemm_emulation_ozii_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_size, vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    ip = ctypes.POINTER(ctypes.c_int)
    sig = {
        "ozgemm_workspace_bytes": (c_size, [c_int, c_int, c_int, c_int]),
        "ozgemm_config": (c_int, [c_int, c_int, c_int, c_int, vp, vp, c_size]),
        "ozgemm_set_stream": (c_int, [vp]),
        "ozgemm_set_panels": (c_int, [c_int]),
        "ozgemm_free": (c_int, []),
        "ozgemm_strerror": (ctypes.c_char_p, [c_int]),
        "ozgemm_dgemm": (c_int, [c_int, c_int, c_int, vp, c_int, vp, c_int, vp, c_int, c_int]),
        "ozgemm_dgemm_noalloc": (c_int, [c_int, c_int, c_int, vp, c_int, vp, c_int, vp, c_int, c_int, vp]),
        "ozgemm_moduli": (c_int, [c_int, ip]),
        "ozgemm_kbits": (c_int, [c_int, c_int]),
        "ozgemm_plane_dims": (c_int, [c_int, c_int, c_int, ip, ip, ip]),
        "ozgemm_stage_scale": (c_int, [c_int, c_int, c_int, c_int, vp, c_int, vp, c_int, vp, vp]),
        "ozgemm_set_bound": (c_int, [c_int]),
        "ozgemm_bound_budget": (c_int, [c_int, c_int, c_int, ip, ip]),
        "ozgemm_stage_residue": (c_int, [c_int, c_int, c_int, c_int, vp, c_int, vp, c_int, vp, vp, vp, vp, vp, vp]),
        "ozgemm_stage_gemm": (c_int, [c_int, c_int, c_int, c_int, vp, vp, vp, vp]),
        "ozgemm_stage_crt": (c_int, [c_int, c_int, c_int, c_int, vp, vp, vp, vp, c_int]),
        "ozgemm_gemm_parts": (c_int, [c_int, c_int, c_int, c_int, ip]),
        "ozgemm_timing": (c_int, [c_int]),
        "ozgemm_phase_ms": (c_int, [ctypes.POINTER(ctypes.c_double), ip]),
        "ozgemm_phase_calls": (c_int, [ctypes.POINTER(ctypes.c_double), c_int, ip]),
        "ozgemm_mfma_ceiling": (c_int, [c_int, c_int, ctypes.c_uint, vp, vp]),
        "ozgemm_scheme1_beta": (c_int, [c_int]),
        "ozgemm_scheme1_outputs": (c_int, [c_int, c_int, c_int]),
        "ozgemm_scheme1_workspace_bytes": (c_size, [c_int, c_int, c_int, c_int, c_int]),
        "ozgemm_scheme1_dgemm": (c_int, [c_int, c_int, c_int, vp, c_int, vp, c_int, vp, c_int, c_int, c_int]),
        "ozgemm_scheme1_stage_split": (c_int, [c_int, c_int, c_int, c_int, c_int, vp, c_int, vp, c_int, vp, vp, vp,
                                               vp]),
        "ozgemm_scheme1_stage_products": (c_int, [c_int, c_int, c_int, c_int, c_int, vp, vp, vp]),
        "ozgemm_scheme1_stage_accumulate": (c_int, [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _ptr(x):
    """Device pointer of a tensor, an int address, or None (NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _check(status: int, where: str) -> int:
    if status != OZGEMM_OK:
        raise OzgemmError(status, where)
    return status


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# --------------------------------------------------------------------------
# host-only
# --------------------------------------------------------------------------

def ozgemm_strerror(status: int) -> str:
    return lib().ozgemm_strerror(status).decode()


def ozgemm_workspace_bytes(max_m: int, max_n: int, max_q: int, s_max: int) -> int:
    return int(lib().ozgemm_workspace_bytes(max_m, max_n, max_q, s_max))


def ozgemm_moduli(s: int) -> list[int]:
    buf = (ctypes.c_int * max(s, 1))()
    _check(lib().ozgemm_moduli(s, buf), "ozgemm_moduli")
    return list(buf)[:s]


def ozgemm_kbits(s: int, q: int) -> int:
    """Returns k (negative when no bits are left); never raises."""
    return int(lib().ozgemm_kbits(s, q))


def ozgemm_plane_dims(m: int, n: int, q: int):
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().ozgemm_plane_dims(m, n, q, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "ozgemm_plane_dims")
    return a.value, b.value, c.value


# --------------------------------------------------------------------------
# configuration
# --------------------------------------------------------------------------

def ozgemm_config(s_max: int, max_m: int, max_n: int, max_q: int, stream=None, workspace=None,
                  workspace_bytes: int | None = None, scheme1_k: int = 0, scheme1_variant: int = OZGEMM_S1_RN) -> int:
    """Configure the library.  With ``workspace=None`` a torch uint8 device
    tensor of ``ozgemm_workspace_bytes(...)`` bytes is allocated and kept
    alive here -- or of ``ozgemm_scheme1_workspace_bytes(max_m, max_n, max_q,
    scheme1_k, scheme1_variant)`` bytes when ``scheme1_k`` > 0 and that is
    larger."""
    global _workspace
    need = ozgemm_workspace_bytes(max_m, max_n, max_q, s_max)
    if scheme1_k > 0:
        need = max(need, ozgemm_scheme1_workspace_bytes(max_m, max_n, max_q, scheme1_k, scheme1_variant))
    hs = _stream(stream)
    if workspace is None:
        import torch
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        workspace_bytes = need
    elif workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().ozgemm_config(s_max, max_m, max_n, max_q, hs, _ptr(workspace), workspace_bytes)
    _check(st, "ozgemm_config")  # on failure the previous configuration and its workspace stay
    _release_workspace()
    _workspace = workspace
    return st


def _release_workspace():
    """Drop the workspace reference held here, after every kernel queued on
    the device has finished: the configured stream may differ from the one the
    tensor was allocated on, and the caching allocator would otherwise hand
    the bytes to new work while queued calls still read and write them."""
    global _workspace
    if _workspace is not None:
        import torch
        torch.cuda.synchronize()
    _workspace = None


def ozgemm_set_stream(stream=None) -> int:
    """Later calls go on `stream`.  Work already queued on the previous stream
    is not ordered before them: the caller orders the two streams."""
    return _check(lib().ozgemm_set_stream(_stream(stream)), "ozgemm_set_stream")


def ozgemm_set_panels(panels: int) -> int:
    """Column panels of the ozgemm_dgemm pipeline: 0 or 1 no pipeline (the
    default), 2..OZGEMM_PANELS_MAX that many panels where the shape allows."""
    return _check(lib().ozgemm_set_panels(panels), "ozgemm_set_panels")


def ozgemm_free() -> int:
    st = lib().ozgemm_free()
    _release_workspace()
    return st


# --------------------------------------------------------------------------
# compute (raw C-ABI signatures; matrices are column-major device buffers)
# --------------------------------------------------------------------------

def ozgemm_dgemm(m, n, q, A, lda, B, ldb, C, ldc, s, check: bool = True) -> int:
    st = lib().ozgemm_dgemm(m, n, q, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, s)
    return _check(st, "ozgemm_dgemm") if check else st


def ozgemm_dgemm_noalloc(m, n, q, A, lda, B, ldb, C, ldc, s, stream=None, check: bool = True) -> int:
    st = lib().ozgemm_dgemm_noalloc(m, n, q, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, s, _stream(stream))
    return _check(st, "ozgemm_dgemm_noalloc") if check else st


def ozgemm_stage_scale(m, n, q, s, A, lda, B, ldb, e, f, check: bool = True) -> int:
    st = lib().ozgemm_stage_scale(m, n, q, s, _ptr(A), lda, _ptr(B), ldb, _ptr(e), _ptr(f))
    return _check(st, "ozgemm_stage_scale") if check else st


def ozgemm_stage_residue(m, n, q, s, A, lda, B, ldb, e, f, Ares, Bres, Aprime=None, Bprime=None,
                         check: bool = True) -> int:
    st = lib().ozgemm_stage_residue(m, n, q, s, _ptr(A), lda, _ptr(B), ldb, _ptr(e), _ptr(f), _ptr(Ares),
                                    _ptr(Bres), _ptr(Aprime), _ptr(Bprime))
    return _check(st, "ozgemm_stage_residue") if check else st


def ozgemm_stage_gemm(m, n, q, s, Ares, Bres, Ct=None, rt=None, check: bool = True) -> int:
    st = lib().ozgemm_stage_gemm(m, n, q, s, _ptr(Ares), _ptr(Bres), _ptr(Ct), _ptr(rt))
    return _check(st, "ozgemm_stage_gemm") if check else st


def ozgemm_stage_crt(m, n, q, s, rt, e, f, C, ldc, check: bool = True) -> int:
    st = lib().ozgemm_stage_crt(m, n, q, s, _ptr(rt), _ptr(e), _ptr(f), _ptr(C), ldc)
    return _check(st, "ozgemm_stage_crt") if check else st


def ozgemm_gemm_parts(m: int, n: int, q: int, s: int) -> int:
    """K parts of the residue-only product of an m x n x q call (needs a device)."""
    p = ctypes.c_int()
    _check(lib().ozgemm_gemm_parts(m, n, q, s, ctypes.byref(p)), "ozgemm_gemm_parts")
    return p.value


def ozgemm_set_bound(mode: int) -> int:
    return _check(lib().ozgemm_set_bound(mode), "ozgemm_set_bound")


def ozgemm_bound_budget(s: int, q: int, mode: int):
    """(kappa_A, kappa_B) of the bit budget, or raises."""
    a, b = ctypes.c_int(), ctypes.c_int()
    _check(lib().ozgemm_bound_budget(s, q, mode, ctypes.byref(a), ctypes.byref(b)), "ozgemm_bound_budget")
    return a.value, b.value


def ozgemm_scheme1_beta(q: int) -> int:
    return lib().ozgemm_scheme1_beta(q)


def ozgemm_scheme1_outputs(k: int, variant: int, q: int) -> int:
    return lib().ozgemm_scheme1_outputs(k, variant, q)


def ozgemm_scheme1_workspace_bytes(m: int, n: int, q: int, k: int, variant: int) -> int:
    return lib().ozgemm_scheme1_workspace_bytes(m, n, q, k, variant)


def ozgemm_scheme1_dgemm(m, n, q, A, lda, B, ldb, C, ldc, k, variant=OZGEMM_S1_RN, check: bool = True) -> int:
    st = lib().ozgemm_scheme1_dgemm(m, n, q, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, k, variant)
    return _check(st, "ozgemm_scheme1_dgemm") if check else st


def ozgemm_scheme1_stage_split(m, n, q, k, variant, A, lda, B, ldb, Aslices, Bslices, gA, gB,
                               check: bool = True) -> int:
    st = lib().ozgemm_scheme1_stage_split(m, n, q, k, variant, _ptr(A), lda, _ptr(B), ldb, _ptr(Aslices),
                                          _ptr(Bslices), _ptr(gA), _ptr(gB))
    return _check(st, "ozgemm_scheme1_stage_split") if check else st


def ozgemm_scheme1_stage_products(m, n, q, k, variant, Aslices, Bslices, P, check: bool = True) -> int:
    st = lib().ozgemm_scheme1_stage_products(m, n, q, k, variant, _ptr(Aslices), _ptr(Bslices), _ptr(P))
    return _check(st, "ozgemm_scheme1_stage_products") if check else st


def ozgemm_scheme1_stage_accumulate(m, n, q, k, variant, P, gA, gB, C, ldc, check: bool = True) -> int:
    st = lib().ozgemm_scheme1_stage_accumulate(m, n, q, k, variant, _ptr(P), _ptr(gA), _ptr(gB), _ptr(C), ldc)
    return _check(st, "ozgemm_scheme1_stage_accumulate") if check else st


def ozgemm_timing(enable: bool) -> int:
    return _check(lib().ozgemm_timing(1 if enable else 0), "ozgemm_timing")


def ozgemm_phase_ms():
    """Returns ([scale, residue, gemm, crt] total milliseconds, calls)."""
    buf = (ctypes.c_double * 4)()
    calls = ctypes.c_int()
    _check(lib().ozgemm_phase_ms(buf, ctypes.byref(calls)), "ozgemm_phase_ms")
    return list(buf), calls.value


def ozgemm_mfma_ceiling(blocks: int, steps: int, seed: int, sink, stream=None, check: bool = True) -> int:
    """Launch the int8 matrix-core rate probe (asynchronous on `stream`, a
    torch stream or None for the current one); sink: int32 device tensor of
    at least 4 * blocks elements."""
    import torch
    if sink.numel() < 4 * blocks or sink.element_size() != 4 or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous 4-byte tensor of at least 4 * blocks elements")
    s = stream if stream is not None else torch.cuda.current_stream()
    st = lib().ozgemm_mfma_ceiling(blocks, steps, seed & 0xFFFFFFFF, _ptr(sink), s.cuda_stream)
    return _check(st, "ozgemm_mfma_ceiling") if check else st


def ozgemm_phase_calls():
    """Per-call phase times: a list of [scale, residue, gemm, crt] ms, one per
    timed call."""
    calls = ctypes.c_int()
    _check(lib().ozgemm_phase_calls(None, 0, ctypes.byref(calls)), "ozgemm_phase_calls")
    n = calls.value
    buf = (ctypes.c_double * max(4 * n, 1))()
    _check(lib().ozgemm_phase_calls(buf, n, ctypes.byref(calls)), "ozgemm_phase_calls")
    return [list(buf[4 * c:4 * c + 4]) for c in range(n)]
