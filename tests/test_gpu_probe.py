"""The int8 matrix-core rate probe (ozgemm_mfma_ceiling) computes the
products it claims to: each wavefront's XOR of its accumulator words equals
the XOR of steps x (A_i B_j^T) over its 4 x 8 tiles, evaluated here in numpy
from the same pseudo-random operand words.  Lane l of a 16x16x64 int8 MFMA
supplies 16 bytes of row l mod 16 (A) or column l mod 16 (B) at K chunk
l / 16, the layout the product kernel relies on; the byte order within a
lane is the same for both operands, so the dot products do not depend on
it."""
import numpy as np
import pytest

from fp64_gemm_emulation_ozii_amd import ozgemm as L

from gpu_util import log

pytestmark = pytest.mark.gpu

FA, FB = 4, 8


def lowbias32(x):
    x = np.asarray(x, dtype=np.uint32)
    x = x ^ (x >> np.uint32(16))
    x = x * np.uint32(0x7FEB352D)
    x = x ^ (x >> np.uint32(15))
    x = x * np.uint32(0x846CA68B)
    return x ^ (x >> np.uint32(16))


def expected_sink(blocks: int, steps: int, seed: int) -> np.ndarray:
    base = np.uint32((seed * 0x9E3779B9) & 0xFFFFFFFF)
    out = np.zeros(4 * blocks, dtype=np.uint32)
    f = np.arange(FA + FB, dtype=np.uint32)[:, None, None]
    lane = np.arange(64, dtype=np.uint32)[None, :, None]
    r = np.arange(4, dtype=np.uint32)[None, None, :]
    for g in range(4 * blocks):
        with np.errstate(over="ignore"):
            words = lowbias32(((np.uint32(g) * (FA + FB) + f) * 64 + lane) * 4 + r + base)
        by = words.astype("<u4").view(np.int8).reshape(FA + FB, 64, 16).astype(np.int64)
        # lane l = chunk * 16 + row  ->  [row, chunk * 16 + byte]
        mats = by.reshape(FA + FB, 4, 16, 16).transpose(0, 2, 1, 3).reshape(FA + FB, 16, 64)
        x = np.uint32(0)
        for i in range(FA):
            for j in range(FB):
                P = (steps * (mats[i] @ mats[FA + j].T)) & 0xFFFFFFFF
                x ^= np.bitwise_xor.reduce(P.astype(np.uint32).ravel())
        out[g] = x
    return out


@pytest.mark.parametrize("blocks,steps,seed", [(3, 1, 0), (2, 5, 12345), (1, 4096, 7)])
def test_probe_computes_its_products(blocks, steps, seed):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    log(f"mfma probe blocks={blocks} steps={steps} seed={seed}")
    sink = torch.zeros(4 * blocks, dtype=torch.int32, device="cuda")
    L.ozgemm_mfma_ceiling(blocks, steps, seed, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expected_sink(blocks, steps, seed))
