"""The serial-LDS debug build against the library (GPU).

libsgemm_emu_serial_lds.so is the library built with SGEMM_EMU_SERIAL_LDS: its
N x K plane GEMM runs one tile per workgroup with a single LDS buffer per
operand and a barrier on each side of every K step -- no copies in flight
across a barrier, no buffer ring, no fragment prefetch, no persistence, no
stream-K.  It issues the same split, B copies, fragment reads and MFMAs in the
same order as the pipelined LDS-DMA kernel, so wherever the library runs that
kernel without stream-K the two results must be equal bit for bit: a race in
the pipeline (a buffer overwritten while still read, a copy read before it
landed) would break the equality.  Both libraries are loaded side by side.
"""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

from gpu_util import dev, host

pytestmark = pytest.mark.gpu

i64, ci, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p


@pytest.fixture(scope="module")
def fe():
    import fp32_emulated_gemm_amd as fe
    return fe


@pytest.fixture(scope="module")
def dbg(fe):
    path = os.path.join(os.path.dirname(os.path.abspath(fe.__file__)), "libsgemm_emu_serial_lds.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: run `python -m fp32_emulated_gemm_amd.build`")
    L = ctypes.CDLL(path)
    L.sgemm_emu_presplit_b.argtypes = [i64, i64, i64, vp, i64, vp, vp, vp, i64, ci, vp, i64, ci, vp]
    L.sgemm_emu_linear.argtypes = [i64, i64, i64, vp, i64, vp, vp, vp, i64, vp, ci, vp, i64, ci, vp]
    L.sgemm_emu_ex.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, ci, vp]
    L.sgemm_emu_split_k.argtypes = [i64, i64, i64, ci]
    L.sgemm_emu_version.restype = ctypes.c_char_p
    for n in ("sgemm_emu_presplit_b", "sgemm_emu_linear", "sgemm_emu_ex", "sgemm_emu_split_k"):
        getattr(L, n).restype = ci
    assert b"serial-LDS" in L.sgemm_emu_version()
    # the debug library's own grid rule answers (no stream-K there), not the library's
    assert L.sgemm_emu_split_k(129, 130, 1024, 5) == 1 and fe.sgemm_emu_split_k(129, 130, 1024) > 1
    return L


def _rng(seed):
    return np.random.Generator(np.random.Philox(key=seed))


def _nk_case(fe, M, N, K, seed):
    g = _rng(seed)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    planes = fe.split(dev(np.ascontiguousarray(B.T)))
    return A, B, dev(A), planes


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _same(x, y):
    return np.array_equal(host(x).view(np.uint32), host(y).view(np.uint32))


# shapes the library runs on the pipelined kernel without stream-K and without A
# planes (grids too full for 64 x 64 tiles): one and several tiles per
# workgroup, ragged M and N, the K tail
NK_SHAPES = [(3000, 2600, 192), (2200, 1300, 128), (4096, 1024, 256), (8200, 1030, 64), (4100, 1100, 320)]


@pytest.mark.parametrize("shape", NK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_nk_planes_bitwise(fe, dbg, shape):
    M, N, K = shape
    assert fe.sgemm_emu_split_k(M, N, K) == 1
    A, B, Ad, P = _nk_case(fe, M, N, K, M + 7 * N + K)
    for nb in (5, 3, 1) if M * N < 4_000_000 else (5,):
        print(f"serial-LDS presplit_b {M}x{N}x{K} nbands={nb}", flush=True, file=sys.stderr)
        C1 = torch.full((M, N), float("nan"), device="cuda")
        C2 = torch.full((M, N), float("nan"), device="cuda")
        fe.sgemm_emu_presplit_b(M, N, K, Ad, K, *P, K, fe.SGEMM_EMU_B_NK, C1, N, nb)
        rc = dbg.sgemm_emu_presplit_b(M, N, K, _ptr(Ad), K, *[_ptr(p) for p in P], K, fe.SGEMM_EMU_B_NK,
                                      _ptr(C2), N, nb, None)
        assert rc == 0
        torch.cuda.synchronize()
        assert _same(C1, C2), f"{shape} nbands={nb}"


def test_linear_bias_gelu_bitwise(fe, dbg):
    """The epilogue with bias and GELU on both kernels."""
    M, N, K = 2200, 1300, 128
    A, B, Ad, P = _nk_case(fe, M, N, K, 77)
    bias = dev(_rng(78).standard_normal(N).astype(np.float32))
    for act in (fe.SGEMM_EMU_ACT_NONE, fe.SGEMM_EMU_ACT_GELU):
        print(f"serial-LDS linear {M}x{N}x{K} act={act}", flush=True, file=sys.stderr)
        Y1 = torch.empty((M, N), device="cuda")
        Y2 = torch.empty((M, N), device="cuda")
        fe.sgemm_emu_linear(M, N, K, Ad, K, *P, K, bias, act, Y1, N, 5)
        assert dbg.sgemm_emu_linear(M, N, K, _ptr(Ad), K, *[_ptr(p) for p in P], K, _ptr(bias), act, _ptr(Y2), N,
                                    5, None) == 0
        torch.cuda.synchronize()
        assert _same(Y1, Y2), f"act={act}"


@pytest.mark.parametrize("shape", [(2048, 1000, 512), (1100, 257, 100)], ids=lambda s: "x".join(map(str, s)))
def test_fp32_b_workspace_planes_bitwise(fe, dbg, shape):
    """FP32 B split into N x K' workspace planes (zero past K, A masked past K)."""
    M, N, K = shape
    kpad = (K + 63) // 64 * 64
    assert fe.sgemm_emu_split_k(M, N, kpad) == 1
    g = _rng(M + N + K)
    Ad = dev(g.standard_normal((M, K)).astype(np.float32))
    Bd = dev(g.standard_normal((K, N)).astype(np.float32))
    print(f"serial-LDS FP32 B {M}x{N}x{K}", flush=True, file=sys.stderr)
    C1 = torch.empty((M, N), device="cuda")
    C2 = torch.empty((M, N), device="cuda")
    fe.sgemm_emu_ex(M, N, K, Ad, K, Bd, N, C1, N, 5, fe.SGEMM_EMU_PRESPLIT_B)
    assert dbg.sgemm_emu_ex(M, N, K, _ptr(Ad), K, _ptr(Bd), N, _ptr(C2), N, 5, fe.SGEMM_EMU_PRESPLIT_B, None) == 0
    torch.cuda.synchronize()
    assert _same(C1, C2)
