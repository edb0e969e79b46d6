"""GPU parity on the five workloads at their full sizes, in the launch
configuration the benchmark times.  Small workloads are compared in full;
large ones on seeded sample rows that the oracle computes one by one."""
import sys

import numpy as np
import pytest
import torch

import workloads
from gpu_util import check_against_fp64, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fe():
    import fp32_emulated_gemm_amd as fe
    return fe


def log(msg):
    print(msg, flush=True, file=sys.stderr)


def gpu_gemm(fe, Ad, Bd, M, N, K, nbands=5, presplit=False, weight_nk=None):
    """presplit=True: planes of B (K x N); weight_nk: B^T as a [N][K] weight, split
    into N x K planes (the benchmark's configuration)."""
    Cd = torch.empty((M, N), dtype=torch.float32, device="cuda")
    if weight_nk is not None:
        planes = [torch.empty((N, K), dtype=torch.int16, device="cuda") for _ in range(3)]
        fe.split_f32_bf16x3(N, K, weight_nk, K, *planes, K)
        fe.sgemm_emu_presplit_b(M, N, K, Ad, K, *planes, K, fe.SGEMM_EMU_B_NK, Cd, N, nbands)
    elif presplit:
        planes = [torch.empty((K, N), dtype=torch.int16, device="cuda") for _ in range(3)]
        fe.split_f32_bf16x3(K, N, Bd, N, *planes, N)
        fe.sgemm_emu_presplit_b(M, N, K, Ad, K, *planes, N, fe.SGEMM_EMU_B_KN, Cd, N, nbands)
    elif nbands == 5:
        fe.sgemm_bf16x9(M, N, K, Ad, K, Bd, N, Cd, N)
    else:
        fe.sgemm_emu(M, N, K, Ad, K, Bd, N, Cd, N, nbands)
    return Cd


def sample_rows(M, n, seed, must=()):
    g = np.random.Generator(np.random.Philox(key=seed))
    rows = set(int(r) for r in g.choice(M, size=min(n, M), replace=False))
    rows.update([0, M - 1, *must])
    return np.array(sorted(rows), dtype=np.int64)


def test_square256_full(fe, orc):
    w = workloads.square256()
    A, B = w["A"], w["B"]
    log("square256")
    C = host(gpu_gemm(fe, dev(A), dev(B), 256, 256, 256))
    check_against_fp64(C, A, B, label="square256")
    E = orc.gemm_emu(A, B)
    assert np.max(np.abs(C.astype(np.float64) - E)) <= 2 * 256 * 2.0 ** -24 * np.max(orc.gemm_f64(A, B)[1])


@pytest.mark.parametrize("presplit", [False, True])
def test_pet_small_full_chain(fe, orc, presplit):
    """X W1, then H = GELU(X W1 in FP64) computed by the oracle, then H W2."""
    w = workloads.pet_small()
    X, W1, W2 = w["X"], w["W1"], w["W2"]
    M = X.shape[0]
    log(f"pet_small presplit={presplit}")
    C1 = host(gpu_gemm(fe, dev(X), dev(W1), M, 1024, 256, presplit=presplit))
    check_against_fp64(C1, X, W1, label="pet_small GEMM1")
    H = orc.gelu_f64_to_f32(orc.gemm_f64(X, W1, want_g=False))
    C2 = host(gpu_gemm(fe, dev(H), dev(W2), M, 256, 1024, presplit=presplit))
    check_against_fp64(C2, H, W2, label="pet_small GEMM2")


def test_square4096_sampled(fe, orc):
    w = workloads.square4096()
    A, B = w["A"], w["B"]
    log("square4096")
    C = host(gpu_gemm(fe, dev(A), dev(B), 4096, 4096, 4096))
    rows = sample_rows(4096, 48, 3)
    check_against_fp64(C[rows], A, B, rows=rows, label="square4096")
    assert np.isfinite(C).all()
    Ct = host(gpu_gemm(fe, dev(A), None, 4096, 4096, 4096, weight_nk=dev(np.ascontiguousarray(B.T))))
    assert np.array_equal(C.view(np.uint32), Ct.view(np.uint32))


def test_pet_large_sampled(fe, orc):
    """The benchmark's configuration: weights held [out][in], split once into N x K
    planes; activations split inside the GEMM."""
    w = workloads.pet_large()
    X, W1, W2, H = w["X"], w["W1"], w["W2"], w["H"]
    M = X.shape[0]
    log("pet_large GEMM1")
    C1 = host(gpu_gemm(fe, dev(X), None, M, 1024, 256, weight_nk=dev(np.ascontiguousarray(W1.T))))
    rows = sample_rows(M, 96, 4)
    check_against_fp64(C1[rows], X, W1, rows=rows, label="pet_large GEMM1")
    assert np.isfinite(C1).all()
    del C1
    log("pet_large GEMM2")
    C2 = host(gpu_gemm(fe, dev(H), None, M, 256, 1024, weight_nk=dev(np.ascontiguousarray(W2.T))))
    check_against_fp64(C2[rows], H, W2, rows=rows, label="pet_large GEMM2")
    assert np.isfinite(C2).all()


def test_stress8192_sampled_with_ablations(fe, orc):
    w = workloads.stress8192()
    A, B = w["A"], w["B"]
    n = 8192
    Ad, Bd = dev(A), dev(B)
    rows = sample_rows(n, 24, 5, must=w["pair_dst"][:8].tolist() + w["pair_src"][:4].tolist())
    log("stress8192 nbands=5")
    C = host(gpu_gemm(fe, Ad, Bd, n, n, n))
    ratio, e_emu, e_naive = check_against_fp64(C[rows], A, B, rows=rows, label="stress8192")
    log(f"stress8192: max ratio to bound {ratio:.3g}, normwise {e_emu:.3g} vs naive {e_naive:.3g}")
    ref, G = orc.gemm_f64(A, B, rows=rows)
    U = 2.0 ** -24
    for nb, bound in [(4, 2.0 ** -30), (3, 2.0 ** -21 + 2.0 ** -30), (2, 2.0 ** -13 + 2.0 ** -21 + 2.0 ** -30)]:
        log(f"stress8192 nbands={nb}")
        Cb = host(gpu_gemm(fe, Ad, Bd, n, n, n, nbands=nb))[rows].astype(np.float64)
        assert np.all(np.abs(Cb - ref) <= (bound + 2 * n * U) * G + 9 * n * 2.0 ** -149)
