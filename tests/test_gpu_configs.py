"""GPU parity on the five workloads at their full sizes, in the launch
configuration the benchmark times.  Every element of every output is checked
against the oracle's FP64 reference (elementwise bound) and the whole output
against the oracle's naive FP32 SGEMM (normwise gate); the large references are
computed in row chunks on the host."""
import sys

import numpy as np
import pytest
import torch

import workloads
from gpu_util import check_against_fp64, check_full, dev, host

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


def test_square4096_full(fe, orc):
    w = workloads.square4096()
    A, B = w["A"], w["B"]
    log("square4096: GPU")
    C = host(gpu_gemm(fe, dev(A), dev(B), 4096, 4096, 4096))
    # the N x K plane path gives the same bits
    Ct = host(gpu_gemm(fe, dev(A), None, 4096, 4096, 4096, weight_nk=dev(np.ascontiguousarray(B.T))))
    assert np.array_equal(C.view(np.uint32), Ct.view(np.uint32))
    log("square4096: every element against the oracle")
    ratio, e, en = check_full("square4096", A, B, C)
    log(f"square4096: max ratio to bound {ratio:.3g}, normwise {e:.3g} vs naive {en:.3g}")


# The large PET system's hidden layer H = fp32(GELU(X W1)) is chained from the
# oracle's FP64 product X W1, built while GEMM 1 is checked, and feeds GEMM 2 on
# both sides (GPU and oracle), so GEMM 2's accuracy is measured on its own.
_PET = {}


def _pet_large():
    if "w" not in _PET:
        _PET["w"] = workloads.pet_large()
    return _PET["w"]


def _pet_large_h(orc, w):
    """H from the chunks of the FP64 reference of X W1 (computed here if the GEMM 1
    test did not already leave it)."""
    if "H" not in _PET:
        X, W1 = w["X"], w["W1"]
        H = np.empty((X.shape[0], W1.shape[1]), dtype=np.float32)
        step = 1 << 15
        for r0 in range(0, X.shape[0], step):
            rows = np.arange(r0, min(X.shape[0], r0 + step), dtype=np.int64)
            H[r0:r0 + rows.size] = orc.gelu_f64_to_f32(orc.gemm_f64(X, W1, rows=rows, want_g=False))
        _PET["H"] = H
    return _PET["H"]


def test_pet_large_gemm1_full(fe, orc):
    """The benchmark's configuration: the weight held [out][in], split once into
    N x K planes; the activations split inside the GEMM."""
    w = _pet_large()
    X, W1 = w["X"], w["W1"]
    M = X.shape[0]
    log("pet_large GEMM1: GPU")
    C1 = host(gpu_gemm(fe, dev(X), None, M, 1024, 256, weight_nk=dev(np.ascontiguousarray(W1.T))))
    H = np.empty((M, 1024), dtype=np.float32)

    def keep(r0, r1, ref):
        H[r0:r1] = orc.gelu_f64_to_f32(ref)

    log("pet_large GEMM1: every element against the oracle")
    ratio, e, en = check_full("pet_large GEMM1", X, W1, C1, keep_ref=keep)
    _PET["H"] = H
    log(f"pet_large GEMM1: max ratio to bound {ratio:.3g}, normwise {e:.3g} vs naive {en:.3g}")


def test_pet_large_gemm2_full_chained(fe, orc):
    """H W2 with H = fp32(GELU(C1_ref)) chained from GEMM 1's FP64 reference."""
    w = _pet_large()
    H, W2 = _pet_large_h(orc, w), w["W2"]
    M = H.shape[0]
    log("pet_large GEMM2: GPU")
    C2 = host(gpu_gemm(fe, dev(H), None, M, 256, 1024, weight_nk=dev(np.ascontiguousarray(W2.T))))
    log("pet_large GEMM2: every element against the oracle")
    ratio, e, en = check_full("pet_large GEMM2", H, W2, C2)
    log(f"pet_large GEMM2: max ratio to bound {ratio:.3g}, normwise {e:.3g} vs naive {en:.3g}")
    _PET.clear()


def test_stress8192_full_with_ablations(fe, orc):
    """All nine products, and the band-drop ablations (8, 6 and 3 products) held to
    their dropped-mass bounds, on every element of the 8192^3 stress workload."""
    w = workloads.stress8192()
    A, B = w["A"], w["B"]
    n = 8192
    Ad, Bd = dev(A), dev(B)
    log("stress8192: GPU, nbands 5, 4, 3, 2")
    C = host(gpu_gemm(fe, Ad, Bd, n, n, n))
    abl = {nb: host(gpu_gemm(fe, Ad, Bd, n, n, n, nbands=nb)) for nb in (4, 3, 2)}
    del Ad, Bd
    log("stress8192: every element against the oracle")
    ratio, e, en = check_full("stress8192", A, B, C, ablations=abl)
    log(f"stress8192: max ratio to bound {ratio:.3g}, normwise {e:.3g} vs naive {en:.3g}")
