"""The benchmark's MFMA-only probe runs the work it is credited with: on
constant operands (every BF16 input 1.0) each lane's sum of its four
accumulators is exactly 4 accumulators x 16 elements x (4 MFMAs x 16
products) per iteration = 4096 per iteration, which fixes the MFMA count
behind sgemm_probe_mfma_flops."""
import ctypes
import os
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def P():
    import fp32_emulated_gemm_amd  # noqa: F401
    P = ctypes.CDLL(os.path.join(ROOT, "fp32_emulated_gemm_amd", "libsgemm_probe.so"))
    P.sgemm_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.sgemm_probe_mfma.restype = ctypes.c_int
    return P


@pytest.mark.parametrize("iters", [1, 10, 123])
def test_constant_operands_exact_sum(P, iters):
    blocks = 4
    print(f"probe constant blocks={blocks} iters={iters}", flush=True, file=sys.stderr)
    out = torch.full((blocks * 512,), float("nan"), dtype=torch.float32, device="cuda")
    assert P.sgemm_probe_mfma(blocks, iters, 0, out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full_like(out, 4096.0 * iters))


def test_random_operands_finite_and_lane_dependent(P):
    blocks = 4
    print(f"probe random blocks={blocks}", flush=True, file=sys.stderr)
    out = torch.full((blocks * 512,), float("nan"), dtype=torch.float32, device="cuda")
    assert P.sgemm_probe_mfma(blocks, 10, 1, out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    assert out.unique().numel() > blocks * 256
