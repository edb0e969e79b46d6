"""The entry point that allocates nothing, against the one it mirrors.

sgemm_emu_presplit_b_noalloc runs the kernels of sgemm_emu_presplit_b with
N x K planes and keeps the stream-K partial results and flags of small tile
grids in a fixed device array instead of allocated workspace.  Called through the C ABI twice in
a row (the second call smaller, so it reuses the array the first one left
behind), each result must equal sgemm_emu_presplit_b's bit for bit, and the
first is also held to the oracle's FP64 bound.
"""
import ctypes
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


def _noalloc(fe):
    L = fe.lib()
    f = L.sgemm_emu_presplit_b_noalloc
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    f.argtypes = [i64, i64, i64, vp, i64, vp, vp, vp, i64, vp, i64, ctypes.c_int, vp]
    f.restype = ctypes.c_int
    return f


def _case(fe, M, N, K, seed):
    g = np.random.Generator(np.random.Philox(key=seed))
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    planes = [torch.empty((N, K), dtype=torch.int16, device="cuda") for _ in range(3)]
    fe.split_f32_bf16x3(N, K, dev(np.ascontiguousarray(B.T)), K, *planes, K)
    return A, B, dev(A), planes


def test_noalloc_matches_presplit_b_twice(fe):
    f = _noalloc(fe)
    stream = torch.cuda.current_stream().cuda_stream
    # both shapes cut their tiles along K (stream-K), so both keep partial
    # results and flags in the fixed array; the second finds the first's there
    for n, (M, N, K, nb) in enumerate([(1024, 512, 2048, 5), (129, 130, 1024, 5), (300, 260, 192, 3)]):
        print(f"noalloc call {n}: {M}x{N}x{K} nbands={nb} split_k={fe.sgemm_emu_split_k(M, N, K, nb)}",
              flush=True, file=sys.stderr)
        A, B, Ad, planes = _case(fe, M, N, K, 900 + n)
        ref = torch.full((M, N), float("nan"), device="cuda")
        fe.sgemm_emu_presplit_b(M, N, K, Ad, K, *planes, K, fe.SGEMM_EMU_B_NK, ref, N, nb)
        out = torch.full((M, N), float("nan"), device="cuda")
        rc = f(M, N, K, Ad.data_ptr(), K, planes[0].data_ptr(), planes[1].data_ptr(), planes[2].data_ptr(), K,
               out.data_ptr(), N, nb, stream)
        assert rc == 0, fe.sgemm_emu_strerror(rc)
        R, C = host(ref), host(out)
        assert np.array_equal(R.view(np.uint32), C.view(np.uint32)), f"call {n}"
        if nb == 5:
            check_against_fp64(C, A, B, label=f"noalloc {M}x{N}x{K}")


def test_noalloc_rejects_before_any_launch(fe):
    f = _noalloc(fe)
    P = 0x10000
    assert f(4, 4, 4, P, 3, P, P, P, 4, P, 4, 5, None) == fe.SGEMM_EMU_EINVAL      # lda < K
    assert f(4, 4, 4, P, 4, P, P, P, 4, P, 4, 6, None) == fe.SGEMM_EMU_EINVAL      # nbands
    assert f(4, 4, 4, P, 4, 0, P, P, 4, P, 4, 5, None) == fe.SGEMM_EMU_ENULL       # null plane
