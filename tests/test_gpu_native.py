"""The library's native FP32 kernel and the performant strategy, through the C ABI.

sgemm_emu_ex with SGEMM_EMU_NATIVE_FP32 runs FP32 products with FP32
accumulation on the FP32 matrix instruction; with SGEMM_EMU_PERFORMANT the
library picks that kernel or the nine-product emulation by shape (the pages'
"performant" strategy; NVIDIA blog, section "BF16x9 on NVIDIA Blackwell GPUs",
Fig. 4).  The native results are held to the same FP64-referenced elementwise
bound and normwise gate as the emulation; where inputs hold Inf or NaN they
follow IEEE FP32 rules, so their class equals the oracle's naive FP32 SGEMM's.
"""
import sys

import numpy as np
import pytest
import torch

from gpu_util import check_against_fp64, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fe():
    import fp32_emulated_gemm_amd as fe
    return fe


def _rng(seed):
    return np.random.Generator(np.random.Philox(key=seed))


def run(fe, A, B, flags, ldc_pad=0, a_offset=0):
    M, K = A.shape
    N = B.shape[1]
    print(f"native M={M} N={N} K={K} flags={flags} ldc_pad={ldc_pad} a_offset={a_offset}", flush=True,
          file=sys.stderr)
    if a_offset:
        buf = np.zeros(M * K + a_offset, np.float32)
        buf[a_offset:] = A.reshape(-1)
        Ad = dev(buf)[a_offset:]
    else:
        Ad = dev(A)
    Bd = dev(B)
    ldc = N + ldc_pad
    Cd = torch.full((max(M, 1) * max(ldc, 1),), float("nan"), dtype=torch.float32, device="cuda")
    fe.sgemm_emu_ex(M, N, K, Ad, max(K, 1), Bd, max(N, 1), Cd, max(ldc, 1), 5, flags)
    C = host(Cd)[: M * ldc].reshape(M, ldc) if M * ldc else np.zeros((M, N), np.float32)
    if ldc_pad:
        assert np.all(np.isnan(C[:, N:])), "padding columns of C were written"
    return C[:, :N]


# shapes covering the native plans on a 256-CU device: 128 x 128 tiles (at
# least one tile per CU), 64 x 64 tiles, 64 x 64 tiles with K slices
SHAPES = [(1, 1, 1), (7, 13, 5), (129, 130, 33), (64, 300, 17), (300, 257, 100), (100, 50, 1000),
          (129, 130, 1024), (6144, 256, 1024), (1024, 1024, 64), (4096, 1024, 512), (2051, 2050, 100)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_native_within_bound_and_deterministic(fe, shape):
    M, N, K = shape
    g = _rng(M * 7 + N * 11 + K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, fe.SGEMM_EMU_NATIVE_FP32)
    check_against_fp64(C, A, B, label=f"native {shape}")
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, fe.SGEMM_EMU_NATIVE_FP32).view(np.uint32))


@pytest.mark.parametrize("shape,a_offset,ldc_pad", [((200, 150, 97), 1, 3), ((257, 129, 64), 3, 0),
                                                     ((130, 131, 67), 0, 5)])
def test_native_scalar_load_path(fe, shape, a_offset, ldc_pad):
    """Unaligned A, N or K not a multiple of 4: the kernel loads one value at a time."""
    M, N, K = shape
    g = _rng(a_offset + ldc_pad + K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, fe.SGEMM_EMU_NATIVE_FP32, ldc_pad=ldc_pad, a_offset=a_offset)
    check_against_fp64(C, A, B, label=f"native scalar {shape}")


def test_native_identity_exact(fe):
    """A = I: every output is one product plus zeros, so C = B exactly."""
    g = _rng(31)
    n = 200
    B = g.standard_normal((n, 170)).astype(np.float32)
    C = run(fe, np.eye(n, dtype=np.float32), B, fe.SGEMM_EMU_NATIVE_FP32)
    assert np.array_equal(C, B)


def test_native_special_values_follow_ieee(fe, orc):
    g = _rng(41)
    M, N, K = 90, 100, 300
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    A[3, 10] = np.inf
    A[4, 11] = -np.inf
    A[5, 12] = np.nan
    B[20, 7] = np.inf
    B[11, :] = 0.0          # A[4, 11] = -Inf meets zeros: NaN in row 4
    C = run(fe, A, B, fe.SGEMM_EMU_NATIVE_FP32)
    E = orc.sgemm_naive_f32(A, B)

    def cls(X):
        return np.where(np.isnan(X), 0, np.where(X == np.inf, 1, np.where(X == -np.inf, 2, 3)))
    assert np.array_equal(cls(C), cls(E))


def test_native_k_zero_and_empty(fe):
    A = np.zeros((5, 0), np.float32)
    B = np.zeros((0, 7), np.float32)
    assert np.array_equal(run(fe, A, B, fe.SGEMM_EMU_NATIVE_FP32), np.zeros((5, 7), np.float32))
    assert run(fe, np.zeros((0, 3), np.float32), np.zeros((3, 4), np.float32), fe.SGEMM_EMU_NATIVE_FP32).size == 0


@pytest.mark.parametrize("shape", [(129, 130, 1024), (1024, 1024, 1024), (6144, 256, 1024), (8192, 8192, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_performant_picks_one_path_and_matches_it(fe, shape):
    """The performant result equals, bit for bit, either the native kernel's or
    the emulation's on the same shape: GEMMs below 2.5e9 flops take the native
    kernel, larger ones the emulation."""
    M, N, K = shape
    g = _rng(K + N)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    P = run(fe, A, B, fe.SGEMM_EMU_PERFORMANT)
    want = run(fe, A, B, fe.SGEMM_EMU_NATIVE_FP32) if 2 * M * N * K < 2.5e9 else run(fe, A, B, 0)
    assert np.array_equal(P.view(np.uint32), want.view(np.uint32))
    check_against_fp64(P, A, B, label=f"performant {shape}")
