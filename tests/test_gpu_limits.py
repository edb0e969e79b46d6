"""Size limits, through the C ABI.

* An output larger than 4 GiB (row offsets past 2^32 bytes): the tile
  descriptors are rebased per tile with 64-bit addresses.
* Leading dimensions at the largest value the header allows (8,388,544
  elements: a 128-row tile span still fits 32-bit byte offsets), for FP32 A
  and for N x K planes of B.  The gaps between rows are filled with NaN, so a
  stray read would poison the result.

Checked against the FP64 oracle (sampled rows of the big output, all rows of
the small ones) and bitwise against the same product with compact layouts.
"""
import sys

import numpy as np
import pytest
import torch

from gpu_util import check_against_fp64, dev, host

pytestmark = pytest.mark.gpu

MAX_LD = (1 << 32) // (128 * 4) - 64      # 8,388,544


@pytest.fixture(scope="module")
def fe():
    import fp32_emulated_gemm_amd as fe
    return fe


def log(msg):
    print(msg, flush=True, file=sys.stderr)


def _rng(seed):
    return np.random.Generator(np.random.Philox(key=seed))


def test_output_beyond_4gib(fe):
    M, N, K = 1_050_097, 1024, 256                 # C: 4.3 GB; rows >= 1,048,576 start past 2^32 bytes
    log(f"limits: output beyond 4 GiB, {M}x{N}x{K}")
    g = torch.Generator(device="cuda").manual_seed(2026)
    Ad = torch.randn((M, K), device="cuda", generator=g)
    B = _rng(77).standard_normal((K, N)).astype(np.float32)
    Bd = dev(B)
    Cd = torch.full((M, N), float("nan"), device="cuda")
    fe.sgemm_bf16x9(M, N, K, Ad, K, Bd, N, Cd, N)
    first_far = (1 << 32) // (4 * N)
    rows = np.unique(np.concatenate([_rng(78).choice(M, 40, replace=False), [0, first_far - 1, first_far],
                                     np.arange(M - 8, M)])).astype(np.int64)
    idx = torch.from_numpy(rows).cuda()
    C_rows = host(Cd.index_select(0, idx))
    A_rows = host(Ad.index_select(0, idx))
    check_against_fp64(C_rows, A_rows, B, label="output beyond 4 GiB")
    # the caller-split N x K planes take the same kernel: bitwise the same
    planes = fe.split(dev(np.ascontiguousarray(B.T)))
    Cd.fill_(float("nan"))
    fe.sgemm_emu_presplit_b(M, N, K, Ad, K, *planes, K, fe.SGEMM_EMU_B_NK, Cd, N, 5)
    assert np.array_equal(host(Cd.index_select(0, idx)).view(np.uint32), C_rows.view(np.uint32))


@pytest.mark.parametrize("M", [130, 1030])
def test_largest_lda(fe, M):
    """FP32 A with lda at the limit (M = 130: B split inside the GEMM; M = 1030:
    the pre-split workspace path), against the oracle and the compact layout."""
    N, K, lda = 96, 64, MAX_LD
    log(f"limits: lda = {lda}, M = {M}")
    g = _rng(90 + M)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    Abuf = torch.full(((M - 1) * lda + K,), float("nan"), device="cuda")
    Abuf.as_strided((M, K), (lda, 1)).copy_(dev(A).reshape(M, K))
    Bd = dev(B)
    C = torch.full((M, N), float("nan"), device="cuda")
    fe.sgemm_emu_ex(M, N, K, Abuf, lda, Bd, N, C, N, 5, fe.SGEMM_EMU_PRESPLIT_B)
    C = host(C)
    check_against_fp64(C, A, B, label=f"lda limit M={M}")
    Cc = torch.full((M, N), float("nan"), device="cuda")
    fe.sgemm_emu_ex(M, N, K, dev(A), K, Bd, N, Cc, N, 5, fe.SGEMM_EMU_PRESPLIT_B)
    assert np.array_equal(C.view(np.uint32), host(Cc).view(np.uint32))


def test_largest_ldb_nk_planes(fe):
    """N x K planes with ldb at the limit (the LDS-DMA kernel) against the oracle
    and against compact planes."""
    M, N, K, ldb = 300, 130, 128, MAX_LD
    log(f"limits: N x K planes with ldb = {ldb}")
    g = _rng(91)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    Bt = dev(np.ascontiguousarray(B.T))
    planes = [torch.full(((N - 1) * ldb + K,), -1, dtype=torch.int16, device="cuda") for _ in range(3)]  # NaN bits
    fe.split_f32_bf16x3(N, K, Bt, K, *planes, ldb)
    Ad = dev(A)
    C = torch.full((M, N), float("nan"), device="cuda")
    fe.sgemm_emu_presplit_b(M, N, K, Ad, K, *planes, ldb, fe.SGEMM_EMU_B_NK, C, N, 5)
    C = host(C)
    check_against_fp64(C, A, B, label="ldb limit")
    compact = fe.split(Bt)
    Cc = torch.full((M, N), float("nan"), device="cuda")
    fe.sgemm_emu_presplit_b(M, N, K, Ad, K, *compact, K, fe.SGEMM_EMU_B_NK, Cc, N, 5)
    assert np.array_equal(C.view(np.uint32), host(Cc).view(np.uint32))
