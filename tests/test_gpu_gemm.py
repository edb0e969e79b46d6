"""GPU GEMM parity against the oracle, through the C ABI (small and ragged sizes).

Bit-exact where the result is unique (identity, permutation, exact-class
inputs, the smallest-band-first case, special-value classes); within the
FP64-referenced bound and the normwise gate elsewhere.
"""
import sys

import numpy as np
import pytest
import torch

from gpu_util import check_against_fp64, dev, exact_class_mask, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fe():
    import fp32_emulated_gemm_amd as fe
    return fe


def _rng(seed):
    return np.random.Generator(np.random.Philox(key=seed))


def run(fe, A, B, nbands=5, entry="fused", ldc_pad=0, a_offset=0):
    """C = A B on the GPU; `entry` picks sgemm_bf16x9/sgemm_emu or the pre-split path."""
    M, K = A.shape
    N = B.shape[1]
    print(f"gemm {entry} M={M} N={N} K={K} nbands={nbands}", flush=True, file=sys.stderr)
    if a_offset:
        buf = np.zeros(M * K + a_offset, np.float32)
        buf[a_offset:] = A.reshape(-1)
        Ad_full = dev(buf)
        Ad = Ad_full[a_offset:]
    else:
        Ad = dev(A)
    Bd = dev(B)
    ldc = N + ldc_pad
    Cd = torch.full((max(M, 1) * max(ldc, 1),), float("nan"), dtype=torch.float32, device="cuda")
    lda = max(K, 1)
    if entry == "presplit":
        planes = [torch.empty(max(K * N, 1), dtype=torch.int16, device="cuda") for _ in range(3)]
        fe.split_f32_bf16x3(K, N, Bd, max(N, 1), *planes, max(N, 1))
        fe.sgemm_emu_presplit_b(M, N, K, Ad, lda, *planes, max(N, 1), fe.SGEMM_EMU_B_KN, Cd, max(ldc, 1), nbands)
    elif entry == "presplit_t":
        Bt = dev(np.ascontiguousarray(B.T))
        planes = [torch.empty(max(K * N, 1), dtype=torch.int16, device="cuda") for _ in range(3)]
        fe.split_f32_bf16x3(N, K, Bt, max(K, 1), *planes, max(K, 1))
        fe.sgemm_emu_presplit_b(M, N, K, Ad, lda, *planes, max(K, 1), fe.SGEMM_EMU_B_NK, Cd, max(ldc, 1), nbands)
    elif entry == "fused_ws":
        fe.sgemm_emu_ex(M, N, K, Ad, lda, Bd, max(N, 1), Cd, max(ldc, 1), nbands, fe.SGEMM_EMU_PRESPLIT_B)
    elif entry == "fused_nows":
        fe.sgemm_emu_ex(M, N, K, Ad, lda, Bd, max(N, 1), Cd, max(ldc, 1), nbands, fe.SGEMM_EMU_NO_WORKSPACE)
    elif entry == "fused_ws_a":
        fe.sgemm_emu_ex(M, N, K, Ad, lda, Bd, max(N, 1), Cd, max(ldc, 1), nbands, fe.SGEMM_EMU_PRESPLIT_A)
    elif nbands == 5 and entry == "fused":
        fe.sgemm_bf16x9(M, N, K, Ad, lda, Bd, max(N, 1), Cd, max(ldc, 1))
    else:
        fe.sgemm_emu(M, N, K, Ad, lda, Bd, max(N, 1), Cd, max(ldc, 1), nbands)
    C = host(Cd)[: M * ldc].reshape(M, ldc) if M * ldc else np.zeros((M, N), np.float32)
    if ldc_pad:
        assert np.all(np.isnan(C[:, N:])), "padding columns of C were written"
    return C[:, :N]


SHAPES = [(1, 1, 1), (7, 13, 5), (128, 128, 32), (129, 130, 33), (64, 300, 17), (300, 257, 100),
          (256, 384, 64), (100, 50, 1000), (31, 33, 257)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("entry", ["fused", "presplit", "presplit_t"])
def test_random_shapes_within_bound(fe, shape, entry):
    M, N, K = shape
    g = _rng(M * 7919 + N * 31 + K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry=entry)
    check_against_fp64(C, A, B, label=f"{entry} {shape}")


# the first four are small enough for 64 x 64 tiles through registers (same bits)
DMA_SHAPES = [(129, 130, 64), (300, 257, 128), (64, 300, 256), (513, 384, 192), (1000, 1030, 1024),
              (4100, 1030, 64), (2500, 2100, 192)]


def same_order_as_fused(fe, M, N, K):
    """True when the N x K plane GEMM adds in the same order as sgemm_bf16x9 on
    FP32 B: neither cuts K (stream-K), or both do it alike (K % 64 == 0 and
    the FP32 B split into N x K planes in a workspace for the same kernel)."""
    fused = fe.sgemm_emu_split_k_fp32_b(M, N, K)
    planes = fe.sgemm_emu_split_k(M, N, K) if K % 64 == 0 else 1
    return (fused == 1 and planes == 1) or (fused > 1 and K % 64 == 0)


@pytest.mark.parametrize("shape", DMA_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_nk_planes_dma_path_within_bound(fe, shape):
    """N x K planes with K a multiple of 64: B copied to LDS by DMA, two steps ahead."""
    M, N, K = shape
    g = _rng(M * 31 + N * 7 + K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="presplit_t")
    check_against_fp64(C, A, B, label=f"nk dma {shape}")
    if same_order_as_fused(fe, M, N, K):
        assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused").view(np.uint32))


@pytest.mark.parametrize("nbands", [1, 2, 3, 4, 5])
def test_nk_planes_dma_path_padded_ldb_and_bands(fe, orc, nbands):
    """Plane rows padded (ldb > K) on the DMA path, every band count, against the
    register path and the oracle's truncated-band value."""
    M, N, K, ldt = 200, 140, 128, 136
    g = _rng(77 + nbands)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    Bt = np.zeros((N, ldt), np.float32)
    Bt[:, :K] = B.T
    Bt[:, K:] = np.inf                                    # padding must never be read
    planes = [torch.empty(N * ldt, dtype=torch.int16, device="cuda") for _ in range(3)]
    fe.split_f32_bf16x3(N, ldt, dev(Bt), ldt, *planes, ldt)
    Cd = torch.empty((M, N), dtype=torch.float32, device="cuda")
    print(f"nk dma padded nbands={nbands}", flush=True, file=sys.stderr)
    fe.sgemm_emu_presplit_b(M, N, K, dev(A), K, *planes, ldt, fe.SGEMM_EMU_B_NK, Cd, N, nbands)
    C = host(Cd).astype(np.float64)
    T = orc.gemm_trunc_f64(A, B, nbands)
    _, G = orc.gemm_f64(A, B)
    assert np.all(np.abs(C - T) <= 2 * K * 2.0 ** -24 * G)
    assert np.array_equal(C.astype(np.float32).view(np.uint32), run(fe, A, B, nbands, "fused").view(np.uint32))


def _fused_in_row_blocks(fe, A, B, nbands):
    """A B from the in-kernel split of FP32 B, one pass over K per tile
    (SGEMM_EMU_NO_WORKSPACE)."""
    return run(fe, A, B, nbands, "fused_nows")


WS_SHAPES = [(1024, 130, 64), (1100, 257, 128), (1500, 1000, 512), (2048, 64, 192),
             (1100, 257, 100), (1024, 130, 33), (1030, 300, 90), (2048, 200, 1000)]   # ragged K: padded planes


@pytest.mark.parametrize("shape", WS_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp32_b_workspace_path(fe, shape):
    """FP32 B with at least 1024 rows of A, pre-split on request: B is split once
    into N x K planes in a workspace (zero-padded to a multiple of 64 in K; the
    kernel masks A past K).  Same result, bit for bit, as sgemm_bf16x9's own
    choice, as the in-kernel split and as the caller-split N x K planes
    (without split-K)."""
    M, N, K = shape
    g = _rng(M + 3 * N + 11 * K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="fused_ws")
    check_against_fp64(C, A, B, label=f"workspace {shape}")
    kpad = (K + 63) // 64 * 64
    if fe.sgemm_emu_split_k_fp32_b(M, N, K) == fe.sgemm_emu_split_k(M, N, kpad):
        assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused").view(np.uint32))
    if K == kpad or fe.sgemm_emu_split_k(M, N, kpad) == 1:
        assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="presplit_t").view(np.uint32))
    if fe.sgemm_emu_split_k(M, N, kpad) == 1:
        assert np.array_equal(C.view(np.uint32), _fused_in_row_blocks(fe, A, B, 5).view(np.uint32))


AB_SHAPES = [(1024, 130, 64), (1100, 257, 128), (1500, 1000, 512), (2048, 64, 192), (1030, 300, 1024),
             (1025, 301, 768)]    # 3 K slices of an odd M N: partials end off a 16-byte boundary


@pytest.mark.parametrize("shape", AB_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp32_a_and_b_workspace_path(fe, shape):
    """SGEMM_EMU_PRESPLIT_A: A is split once into M x K planes beside B's N x K
    planes and the plane kernel copies both (no split in the kernel).  Within
    the FP64 bound, and bit for bit the B-only workspace path (the same split,
    tiles, MFMA order and, on small grids, the same K slices) and the
    in-kernel split of A."""
    M, N, K = shape
    g = _rng(M + 5 * N + 13 * K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="fused_ws_a")
    check_against_fp64(C, A, B, label=f"A and B workspace {shape}")
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused_ws").view(np.uint32))
    if fe.sgemm_emu_split_k(M, N, K) == 1:
        assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="presplit_t").view(np.uint32))


@pytest.mark.parametrize("nbands", [1, 2, 3, 4])
def test_fp32_a_and_b_workspace_path_bands(fe, nbands):
    M, N, K = 1030, 200, 128
    g = _rng(910 + nbands)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, nbands, "fused_ws_a")
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, nbands, "fused_ws").view(np.uint32))


def test_fp32_a_and_b_workspace_path_rne(fe):
    M, N, K = 1100, 260, 256
    g = _rng(920)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    for nbands in (5, 2):
        C = _run_ex(fe, A, B, nbands, fe.SGEMM_EMU_SPLIT_RNE | fe.SGEMM_EMU_PRESPLIT_A)
        W = _run_ex(fe, A, B, nbands, fe.SGEMM_EMU_SPLIT_RNE | fe.SGEMM_EMU_PRESPLIT_B)
        assert np.array_equal(C.view(np.uint32), W.view(np.uint32)), f"nbands={nbands}"


@pytest.mark.parametrize("pad", [4, 5])
def test_fp32_a_and_b_workspace_padded_lda(fe, pad):
    """A with lda = K + pad and NaN in every gap between rows, through the A
    split into workspace planes: the gaps never reach the planes, so the result
    equals the compact layout's bit for bit (pad = 5 also leaves A's rows
    without 16-byte alignment, which the split's scalar path takes)."""
    M, N, K = 1100, 300, 128
    g = _rng(960 + pad)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    lda = K + pad
    Apad = np.full((M, lda), np.nan, np.float32)
    Apad[:, :K] = A
    Cd = torch.empty((M, N), dtype=torch.float32, device="cuda")
    print(f"gemm ex padded lda={lda} M={M} N={N} K={K}", flush=True, file=sys.stderr)
    fe.sgemm_emu_ex(M, N, K, dev(Apad), lda, dev(B), N, Cd, N, 5, fe.SGEMM_EMU_PRESPLIT_A)
    C = host(Cd)
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused_ws_a").view(np.uint32))


@pytest.mark.parametrize("nbands", [5, 3, 1])
def test_fp32_a_and_b_workspace_exact_class_vs_oracle(fe, orc, nbands):
    """Through the plane kernel, elements whose band sums are exact in any order
    equal the oracle emulation bit for bit."""
    g = _rng(930)
    M, N, K = 1024, 36, 64

    def draw(shape):
        m = g.integers(1 << 15, 1 << 16, size=shape).astype(np.float64)
        return (m * np.where(g.integers(0, 2, size=shape) == 1, -1.0, 1.0)).astype(np.float32)

    A, B = draw((M, K)), draw((K, N))
    mask = exact_class_mask(A, B)
    assert mask.mean() > 0.3
    C = run(fe, A, B, nbands, "fused_ws_a")
    E = orc.gemm_emu(A, B, nbands)
    assert np.array_equal(C.view(np.uint32)[mask], E.view(np.uint32)[mask])


def test_presplit_a_rule_at_4096_columns(fe):
    """With N >= 4096 (M >= 1024, K % 64 == 0) A is split into workspace planes
    by default, for FP32 B (sgemm_bf16x9) and beside a caller's N x K planes
    alike: within the bound on sampled rows, and bit for bit the N x K planes
    run in row blocks below 1024 rows, where the kernel splits A itself (each
    block still at least 192 tiles, so no block is cut along K)."""
    M, N, K = 1600, 4096, 192
    g = _rng(940)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="fused")
    rows = np.sort(g.choice(M, size=32, replace=False))
    check_against_fp64(C[rows], A, B, rows=rows, label="A pre-split rule")
    Cnk = run(fe, A, B, entry="presplit_t")
    blocks = np.concatenate([run(fe, A[i:i + 800], B, entry="presplit_t") for i in range(0, M, 800)])
    assert np.array_equal(C.view(np.uint32), Cnk.view(np.uint32))
    assert np.array_equal(C.view(np.uint32), blocks.view(np.uint32))


KN_SHAPES = [(2048, 2048, 2048), (1024, 300, 1024), (1030, 300, 1000), (1100, 4096, 128)]


@pytest.mark.parametrize("shape", KN_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_kn_planes_transposed_into_workspace(fe, shape):
    """K x N planes where the workspace rule holds (2 M N K >= 1.2e10, or a grid
    small enough for split-K): copied, transposed, into N x K' workspace planes
    (zero past K) for the LDS-DMA kernel.  Within the bound on sampled rows and
    bit for bit the FP32 B workspace path, which runs the same kernel, K slices
    and (for N >= 4096) the same A planes."""
    M, N, K = shape
    g = _rng(M + 7 * N + 3 * K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="presplit")
    rows = np.sort(g.choice(M, size=48, replace=False))
    check_against_fp64(C[rows], A, B, rows=rows, label=f"K x N planes {shape}")
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused_ws").view(np.uint32))


@pytest.mark.parametrize("nbands", [1, 3])
def test_kn_planes_transposed_bands(fe, nbands):
    M, N, K = 1024, 300, 1024
    g = _rng(950 + nbands)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    assert np.array_equal(run(fe, A, B, nbands, "presplit").view(np.uint32),
                          run(fe, A, B, nbands, "fused_ws").view(np.uint32))


@pytest.mark.parametrize("nbands", [1, 2, 3, 4])
def test_fp32_b_workspace_path_bands(fe, nbands):
    M, N, K = 1030, 200, 128
    g = _rng(900 + nbands)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, nbands, "fused_ws")
    assert np.array_equal(C.view(np.uint32), _fused_in_row_blocks(fe, A, B, nbands).view(np.uint32))


def test_fp32_b_workspace_ragged_k_masks_a_tail(fe):
    """Ragged K through the padded planes: A's values past K (the next row's
    first elements, here Inf and NaN) must not reach the products."""
    M, N, K = 1024, 96, 100
    g = _rng(515)
    buf = g.standard_normal(M * K + 64).astype(np.float32)
    A = buf[: M * K].reshape(M, K).copy()
    A[1:, :28] = np.where(g.random((M - 1, 28)) < 0.5, np.inf, np.nan)   # row i+1's head follows row i's tail
    A[0, :] = 1.0
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="fused_ws")
    R = _fused_in_row_blocks(fe, A, B, 5)
    assert np.array_equal(np.isnan(C), np.isnan(R)) and np.array_equal(np.isinf(C), np.isinf(R))
    assert np.all(np.isfinite(C[0]))
    fin = np.isfinite(R)
    assert np.array_equal(C[fin].view(np.uint32), R[fin].view(np.uint32))


def test_fp32_b_workspace_path_special_values(fe):
    """Inf, NaN, subnormals and zeros in B take the transposing split's exact path."""
    M, N, K = 1024, 96, 128
    g = _rng(4242)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    B[3, 5] = np.inf
    B[70, 17] = -np.inf
    B[100, 40] = np.nan
    B[9, 60] = np.float32(1e-40)
    B[:, 80] = 0.0
    C = run(fe, A, B, entry="fused_ws")
    R = _fused_in_row_blocks(fe, A, B, 5)
    assert np.array_equal(np.isnan(C), np.isnan(R))
    fin = ~np.isnan(R)
    assert np.array_equal(C[fin].view(np.uint32), R[fin].view(np.uint32))


@pytest.mark.parametrize("shape", [(129, 130, 1024), (513, 384, 192), (1000, 1030, 1024), (64, 300, 100)],
                         ids=lambda s: "x".join(map(str, s)))
def test_no_workspace_one_pass(fe, shape):
    """SGEMM_EMU_NO_WORKSPACE: B split inside the kernel, each tile's whole K in
    one workgroup, on grids the default path cuts along K (stream-K): within
    the bound, deterministic, and bit for bit the default where that does not
    cut K."""
    M, N, K = shape
    g = _rng(M + 17 * N + 5 * K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="fused_nows")
    check_against_fp64(C, A, B, label=f"no workspace {shape}")
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused_nows").view(np.uint32))
    if fe.sgemm_emu_split_k_fp32_b(M, N, K) == 1:
        assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused").view(np.uint32))


PERSIST_SHAPES = [(4100, 1100, 128), (8200, 1030, 64), (4096, 2048, 256)]


@pytest.mark.parametrize("shape", PERSIST_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dma_path_several_tiles_per_workgroup(fe, shape):
    """More tiles than resident workgroups: each workgroup walks several tiles and
    loads the next tile's first K steps during the current tile's last ones."""
    M, N, K = shape
    g = _rng(M + 5 * N + 17 * K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="presplit_t")
    check_against_fp64(C, A, B, label=f"persistent {shape}")
    assert np.array_equal(C.view(np.uint32), _fused_in_row_blocks(fe, A, B, 5).view(np.uint32))
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused").view(np.uint32))


def test_dma_path_special_values_in_next_tile_first_step(fe):
    """Inf and NaN in A at k < 32 of tiles that are not a workgroup's first: their
    first K step is split at the end of the previous tile, on the rare exact path."""
    M, N, K = 8200, 1030, 64
    g = _rng(31337)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    for r, k, v in [(300 * 128 // 9 + 5, 3, np.inf), (5000, 0, -np.inf), (7777, 31, np.nan), (8199, 7, np.inf)]:
        A[r, k] = v
    C = run(fe, A, B, entry="presplit_t")
    R = _fused_in_row_blocks(fe, A, B, 5)
    assert np.array_equal(np.isnan(C), np.isnan(R))
    fin = ~np.isnan(R)
    assert np.array_equal(C[fin].view(np.uint32), R[fin].view(np.uint32))


SPLITK_SHAPES = [(1024, 1024, 1024), (6144, 256, 1024), (129, 130, 1024), (64, 300, 1024), (256, 256, 1024),
                 (700, 40, 2048)]


@pytest.mark.parametrize("shape", SPLITK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_split_k_within_bound_and_deterministic(fe, shape):
    """Small tile grids share their work stream-K style: each piece of a tile
    runs the method on its K range, the pieces' results are added in K order.
    Within the bound, identical on repeat, and sgemm_bf16x9 on FP32 B agrees
    with the caller-split planes bit for bit where it takes the same kernel,
    else (one pass per 64 x 64 tile) with the one-pass result."""
    M, N, K = shape
    assert fe.sgemm_emu_split_k(M, N, K) > 1
    g = _rng(M * 3 + N * 5 + K * 7)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="presplit_t")
    check_against_fp64(C, A, B, label=f"split-k {shape}")
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="presplit_t").view(np.uint32))
    F = run(fe, A, B, entry="fused")
    check_against_fp64(F, A, B, label=f"split-k fused {shape}")
    if fe.sgemm_emu_split_k_fp32_b(M, N, K) > 1:
        # FP32 B split into N x K workspace planes for the same stream-K kernel, at any M
        assert np.array_equal(C.view(np.uint32), F.view(np.uint32))
    else:
        assert np.array_equal(F.view(np.uint32), run(fe, A, B, entry="fused_nows").view(np.uint32))


@pytest.mark.parametrize("shape", [(3072, 1536, 1024), (8192, 640, 1024)], ids=lambda s: "x".join(map(str, s)))
def test_streamk_on_partly_filled_grids(fe, shape):
    """Grids of 1.1-1.3 waves of tiles with long K take stream-K too: fewer
    workgroups than tiles, so runs hold whole tiles between a tile's start and
    another's end.  Within the bound on sampled rows (every tile row), identical
    on repeat, FP32 B equal to the caller's N x K planes bit for bit, and the
    one-pass result (SGEMM_EMU_NO_WORKSPACE) within the same bound."""
    M, N, K = shape
    assert fe.sgemm_emu_split_k(M, N, K) > 1
    g = _rng(M + 3 * N + 5 * K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="presplit_t")
    rows = np.unique(np.concatenate([np.arange(0, M, 128) + g.integers(0, 128, size=(M + 127) // 128),
                                     [M - 1]]).clip(0, M - 1))
    check_against_fp64(C[rows], A, B, rows=rows, label=f"stream-K {shape}")
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="presplit_t").view(np.uint32))
    assert fe.sgemm_emu_split_k_fp32_b(M, N, K) == fe.sgemm_emu_split_k(M, N, K)
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused").view(np.uint32))
    R = run(fe, A, B, entry="fused_nows")
    check_against_fp64(R[rows], A, B, rows=rows, label=f"one pass {shape}")


@pytest.mark.parametrize("nbands", [1, 2, 3, 4, 5])
def test_split_k_bands(fe, orc, nbands):
    M, N, K = 129, 130, 1024
    g = _rng(600 + nbands)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, nbands, "presplit_t").astype(np.float64)
    T = orc.gemm_trunc_f64(A, B, nbands)
    _, G = orc.gemm_f64(A, B)
    assert np.all(np.abs(C - T) <= 2 * K * 2.0 ** -24 * G)


def test_split_k_special_values_class(fe, orc):
    """Inf / NaN through split-K: the class of each output matches the oracle
    emulation's (a NaN or Inf band partial stays NaN or Inf through the slice sums)."""
    g = _rng(19)
    M, N, K = 100, 120, 1024
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    B[700, :] = np.float32(np.pi)
    A[2, 700] = np.inf
    A[5, 700] = -np.inf
    A[7, 10] = np.nan
    B[300, 60] = np.inf
    A[13, 300] = 0.0
    B[700, 4] = 1.0
    assert fe.sgemm_emu_split_k(M, N, K) > 1
    C = run(fe, A, B, entry="presplit_t")
    E = orc.gemm_emu(A, B)

    def cls(X):
        return np.where(np.isnan(X), 0, np.where(X == np.inf, 1, np.where(X == -np.inf, 2, 3)))
    assert np.array_equal(cls(C), cls(E))


@pytest.mark.parametrize("entry", ["fused", "presplit_t"])
def test_split_k_exact_integers_bitwise_vs_oracle(fe, orc, entry):
    """Stream-K on a shape where every partial result is exact: 1024 x 512 x 2048
    (32 tiles of 32 K pairs shared by all CUs, each tile cut into several
    pieces).  A holds 48 nonzero integers per row (|a| < 2^9, so the split puts
    them into bands 0-2), B nonzero integers of the same size.  Each band sum,
    each piece's recombination and the sum of the pieces are then integers below
    2^24, exact in any order, so the GPU result must equal the exact dot product
    and the oracle's one-pass emulation (pieces recombined separately and added
    give the same bits as one recombination over all K)."""
    M, N, K = 1024, 512, 2048
    assert fe.sgemm_emu_split_k(M, N, K) > 1
    g = _rng(2048)
    A = np.zeros((M, K), np.float32)
    for i in range(M):
        cols = g.choice(K, size=48, replace=False)
        A[i, cols] = g.integers(1, 512, size=48) * np.where(g.integers(0, 2, size=48) == 1, -1, 1)
    B = (g.integers(1, 512, size=(K, N)) * np.where(g.integers(0, 2, size=(K, N)) == 1, -1, 1)).astype(np.float32)
    exact = (A.astype(np.int64) @ B.astype(np.int64))
    assert np.abs(exact).max() < 1 << 24
    C = run(fe, A, B, entry=entry)
    E = orc.gemm_emu(A, B)
    assert np.array_equal(E.astype(np.int64), exact)
    assert np.array_equal(C.astype(np.int64), exact)
    nz = exact != 0
    assert np.array_equal(C.view(np.uint32)[nz], E.view(np.uint32)[nz])


TILE64_SHAPES = [(1024, 1024, 1000), (6144, 256, 1000), (1025, 301, 768), (777, 555, 333), (513, 384, 192),
                 (17, 33, 5)]


@pytest.mark.parametrize("shape", TILE64_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp32_b_on_64_tiles(fe, shape):
    """Partly filled grids of FP32 B that the cost model gives to the one-pass
    kernel on 64 x 64 tiles (B split inside each tile, nothing allocated):
    within the FP64 bound, identical on repeat, bit for bit the caller's K x N
    planes (the same choice, N even) and the caller's N x K planes where those run one
    pass over K on 128 x 128 tiles (same split, products and MFMA order per
    output).  Ragged M, N and K."""
    M, N, K = shape
    kpad = (K + 63) // 64 * 64
    assert fe.sgemm_emu_split_k_fp32_b(M, N, K) == 1
    g = _rng(M + 7 * N + 3 * K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="fused")
    check_against_fp64(C, A, B, label=f"64 x 64 tiles {shape}")
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused").view(np.uint32))
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused_nows").view(np.uint32))
    # K x N planes read as column pairs (N even) follow FP32 B's choice
    if N % 2 == 0:
        assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="presplit").view(np.uint32))
    if K % 64 != 0 or fe.sgemm_emu_split_k(M, N, K) == 1:
        assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="presplit_t").view(np.uint32))
    if fe.sgemm_emu_split_k(M, N, kpad) > 1:
        # the cost model preferred these tiles to stream-K: the caller's planes still take it
        check_against_fp64(run(fe, A, B, entry="presplit_t"), A, B, label=f"stream-K beside {shape}")


@pytest.mark.parametrize("nbands", [1, 2, 3, 4])
def test_fp32_b_on_64_tiles_bands_offsets_and_ldc(fe, orc, nbands):
    """The 64 x 64 kernel for every band count, with A off its 16-byte
    alignment (element loads) and C rows padded: the oracle's truncated-band
    value within its bound, and the caller's planes on 128 x 128 tiles bit for
    bit."""
    M, N, K = 777, 555, 333
    assert fe.sgemm_emu_split_k_fp32_b(M, N, K) == 1
    g = _rng(4000 + nbands)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, nbands, "fused", ldc_pad=3, a_offset=1).astype(np.float64)
    T = orc.gemm_trunc_f64(A, B, nbands)
    _, G = orc.gemm_f64(A, B)
    assert np.all(np.abs(C - T) <= 2 * K * 2.0 ** -24 * G)
    R = run(fe, A, B, nbands, "presplit_t")
    assert np.array_equal(C.astype(np.float32).view(np.uint32), R.view(np.uint32))


def test_fp32_b_on_64_tiles_exact_integers_and_specials(fe, orc):
    """1024^3 on 64 x 64 tiles (where 128 x 128 tiles would take stream-K):
    integer operands whose every partial sum is exact give the exact product,
    as the oracle's emulation does; Inf and NaN in A and B give the oracle
    emulation's class for every output."""
    M = N = K = 1024
    assert fe.sgemm_emu_split_k_fp32_b(M, N, K) == 1 and fe.sgemm_emu_split_k(M, N, K) > 1
    g = _rng(6464)
    A = np.zeros((M, K), np.float32)
    for i in range(M):
        cols = g.choice(K, size=48, replace=False)
        A[i, cols] = g.integers(1, 512, size=48) * np.where(g.integers(0, 2, size=48) == 1, -1, 1)
    B = (g.integers(1, 512, size=(K, N)) * np.where(g.integers(0, 2, size=(K, N)) == 1, -1, 1)).astype(np.float32)
    exact = A.astype(np.int64) @ B.astype(np.int64)
    assert np.abs(exact).max() < 1 << 24
    C = run(fe, A, B, entry="fused")
    assert np.array_equal(C.astype(np.int64), exact)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    A[3, 700], A[900, 5], A[1023, 1023] = np.inf, -np.inf, np.nan
    B[700, 64], B[12, 1000] = np.inf, np.nan
    B[:, 513] = 0.0
    C = run(fe, A, B, entry="fused")
    E = orc.gemm_emu(A, B)

    def cls(X):
        return np.where(np.isnan(X), 0, np.where(X == np.inf, 1, np.where(X == -np.inf, 2, 3)))
    assert np.array_equal(cls(C), cls(E))


def test_fp32_b_on_64_tiles_rne(fe, orc):
    """SGEMM_EMU_SPLIT_RNE on 64 x 64 tiles: within the bound against the
    oracle's RNE truncated-band value, and bit for bit the one pass on
    128 x 128 tiles that SGEMM_EMU_PRESPLIT_B leaves to rows >= 1024 when K
    is not a multiple of 64 (the RNE split is not padded into planes)."""
    M, N, K = 1025, 301, 700
    assert fe.sgemm_emu_split_k_fp32_b(M, N, K) == 1
    g = _rng(6565)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    rows = np.sort(g.choice(M, size=96, replace=False))
    _, G = orc.gemm_f64(A, B, rows=rows)
    for nb in (5, 2):
        C = _run_ex(fe, A, B, nb, fe.SGEMM_EMU_SPLIT_RNE)
        T = orc.gemm_trunc_f64(A, B, nb, rows=rows, flags=orc.ORC_SPLIT_RNE)
        assert np.all(np.abs(C[rows].astype(np.float64) - T) <= 2 * K * 2.0 ** -24 * G), f"nbands={nb}"
        R = _run_ex(fe, A, B, nb, fe.SGEMM_EMU_SPLIT_RNE | fe.SGEMM_EMU_PRESPLIT_B)
        assert np.array_equal(C.view(np.uint32), R.view(np.uint32)), f"nbands={nb}"


NK64_SHAPES = [(1024, 1024, 512), (2048, 512, 512), (513, 384, 192), (777, 555, 333)]


@pytest.mark.parametrize("shape", NK64_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_nk_planes_on_64_tiles(fe, shape):
    """The caller's N x K planes on a partly filled grid that stream-K leaves
    alone (or cannot take: K % 64 != 0) run one pass per 64 x 64 tile: within
    the bound, bit for bit the K x N planes' one pass on 128 x 128 tiles and
    FP32 B, and the entry point that allocates nothing gives the same bits."""
    M, N, K = shape
    assert fe.sgemm_emu_split_k(M, N, K) == 1 and fe.sgemm_emu_split_k_fp32_b(M, N, K) == 1
    g = _rng(M + 11 * N + 5 * K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="presplit_t")
    check_against_fp64(C, A, B, label=f"N x K planes, 64 x 64 tiles {shape}")
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="presplit").view(np.uint32))
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused").view(np.uint32))
    P = fe.split(dev(np.ascontiguousarray(B.T)))
    Cn = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    print(f"noalloc {M}x{N}x{K}", flush=True, file=sys.stderr)
    fe.sgemm_emu_presplit_b_noalloc(M, N, K, dev(A), K, *P, K, Cn, N, 5)
    assert np.array_equal(C.view(np.uint32), host(Cn).view(np.uint32))


@pytest.mark.parametrize("shape", [(1100, 900, 700), (4100, 1100, 700), (300, 257, 100)],
                         ids=lambda s: "x".join(map(str, s)))
def test_nk_planes_even_k_word_loads(fe, shape):
    """N x K planes whose K is even but not a multiple of 8 (ldb = K) load B
    two elements at a time, on 64 x 64 and on 128 x 128 tiles: within the
    bound and bit for bit the one pass over FP32 B (SGEMM_EMU_NO_WORKSPACE)."""
    M, N, K = shape
    assert K % 2 == 0 and K % 8 != 0
    g = _rng(M + 3 * N + 7 * K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="presplit_t")
    rows = None if M * N * K < 1e9 else np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    check_against_fp64(C if rows is None else C[rows], A, B, rows=rows, label=f"N x K word loads {shape}")
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused_nows").view(np.uint32))


def _sweep_shapes(n=20):
    g = np.random.Generator(np.random.Philox(key=2718))
    out = []
    for _ in range(n):
        M, N = (int(x) for x in g.integers(1, 700, size=2))
        K = int(g.integers(1, 1500)) if g.integers(0, 2) else int(g.integers(1, 24)) * 64
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("shape", _sweep_shapes(), ids=lambda s: "x".join(map(str, s)))
def test_dispatch_sweep_bound_and_consistency(fe, shape):
    """Seeded random shapes across the dispatch rules (one pass on 128 x 128 or
    64 x 64 tiles, stream-K, pre-split or not): every B source within the FP64
    bound, and the bit equalities the query calls promise -- FP32 B with one
    pass equals SGEMM_EMU_NO_WORKSPACE, K x N planes with N even equal FP32 B,
    N x K planes equal FP32 B where both cut K alike."""
    M, N, K = shape
    g = _rng(M * 7919 + N * 31 + K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    F = run(fe, A, B, entry="fused")
    check_against_fp64(F, A, B, label=f"sweep fused {shape}")
    KN = run(fe, A, B, entry="presplit")
    NK = run(fe, A, B, entry="presplit_t")
    W = run(fe, A, B, entry="fused_nows")
    for name, X in (("K x N", KN), ("N x K", NK), ("no workspace", W)):
        check_against_fp64(X, A, B, label=f"sweep {name} {shape}", normwise=False)
    if fe.sgemm_emu_split_k_fp32_b(M, N, K) == 1:
        assert np.array_equal(F.view(np.uint32), W.view(np.uint32))
    if N % 2 == 0:
        assert np.array_equal(F.view(np.uint32), KN.view(np.uint32))
    if same_order_as_fused(fe, M, N, K):
        assert np.array_equal(F.view(np.uint32), NK.view(np.uint32))


@pytest.mark.parametrize("shape", [(128, 128, 32768), (200, 70, 20000), (64, 1000, 8192)],
                         ids=lambda s: "x".join(map(str, s)))
def test_long_k_small_grids(fe, shape):
    """Few tiles and a long K: stream-K cuts each tile into its most pieces
    (at most 8), with K padded for FP32 B where it is not a multiple of 64.
    Every B source within the bound and identical on repeat; FP32 B, K x N and
    N x K planes bit for bit where the query calls say they cut K alike."""
    M, N, K = shape
    kpad = (K + 63) // 64 * 64
    assert fe.sgemm_emu_split_k_fp32_b(M, N, K) == fe.sgemm_emu_split_k(M, N, kpad) > 1
    g = _rng(M + N + K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    F = run(fe, A, B, entry="fused")
    check_against_fp64(F, A, B, label=f"long K fused {shape}")
    assert np.array_equal(F.view(np.uint32), run(fe, A, B, entry="fused").view(np.uint32))
    KN = run(fe, A, B, entry="presplit")
    check_against_fp64(KN, A, B, label=f"long K K x N {shape}", normwise=False)
    if N % 2 == 0:
        assert np.array_equal(F.view(np.uint32), KN.view(np.uint32))
    NK = run(fe, A, B, entry="presplit_t")
    check_against_fp64(NK, A, B, label=f"long K N x K {shape}", normwise=False)
    if same_order_as_fused(fe, M, N, K):
        assert np.array_equal(F.view(np.uint32), NK.view(np.uint32))


def test_presplit_equals_fused_bitwise(fe):
    g = _rng(5)
    A = g.standard_normal((200, 150)).astype(np.float32)
    B = g.standard_normal((150, 190)).astype(np.float32)
    for nb in (1, 3, 5):
        ref = run(fe, A, B, nb, "fused").view(np.uint32)
        assert np.array_equal(ref, run(fe, A, B, nb, "presplit").view(np.uint32))
        if same_order_as_fused(fe, 200, 190, 150):   # else FP32 B and K x N planes take stream-K
            assert np.array_equal(ref, run(fe, A, B, nb, "presplit_t").view(np.uint32))
    # the one-pass kernels agree
    for nb in (1, 5):
        ref = run(fe, A, B, nb, "fused_nows").view(np.uint32)
        assert np.array_equal(ref, run(fe, A, B, nb, "presplit_t").view(np.uint32))


def test_unaligned_a_and_padded_c(fe):
    """A at a 4-byte (not 16-byte) offset takes the scalar-load path; C with
    ldc > N leaves the padding untouched."""
    g = _rng(6)
    A = g.standard_normal((70, 45)).astype(np.float32)
    B = g.standard_normal((45, 66)).astype(np.float32)
    C1 = run(fe, A, B, a_offset=1, ldc_pad=3)
    C0 = run(fe, A, B)
    check_against_fp64(C1, A, B, label="unaligned")
    assert np.array_equal(C0.view(np.uint32), C1.view(np.uint32))


@pytest.mark.parametrize("entry", ["fused", "presplit", "presplit_t"])
@pytest.mark.parametrize("M,N,K,lda", [(70, 66, 45, 48), (129, 131, 61, 64), (40, 30, 5, 8)])
def test_ragged_k_with_padded_lda(fe, entry, M, N, K, lda):
    """K not a multiple of the 8-wide staging chunks with lda > K: the elements
    past K in each row of A are other data and must not contribute."""
    g = _rng(M + N + K)
    Abuf = g.standard_normal((M, lda)).astype(np.float32) * 1e3     # junk past K
    A = np.ascontiguousarray(Abuf[:, :K])
    B = g.standard_normal((K, N)).astype(np.float32)
    Ad = dev(Abuf)
    Bd = dev(B)
    Cd = torch.empty((M, N), dtype=torch.float32, device="cuda")
    print(f"ragged K {entry} M={M} N={N} K={K} lda={lda}", flush=True, file=sys.stderr)
    if entry == "fused":
        fe.sgemm_bf16x9(M, N, K, Ad, lda, Bd, N, Cd, N)
    elif entry == "presplit":
        planes = [torch.empty(K * N, dtype=torch.int16, device="cuda") for _ in range(3)]
        fe.split_f32_bf16x3(K, N, Bd, N, *planes, N)
        fe.sgemm_emu_presplit_b(M, N, K, Ad, lda, *planes, N, fe.SGEMM_EMU_B_KN, Cd, N, 5)
    else:
        ldt = K + 3
        Bt = np.zeros((N, ldt), np.float32)
        Bt[:, :K] = B.T
        Bt[:, K:] = 7e3                                                   # junk past K in each plane row
        planes = [torch.empty(N * ldt, dtype=torch.int16, device="cuda") for _ in range(3)]
        fe.split_f32_bf16x3(N, ldt, dev(Bt), ldt, *planes, ldt)
        fe.sgemm_emu_presplit_b(M, N, K, Ad, lda, *planes, ldt, fe.SGEMM_EMU_B_NK, Cd, N, 5)
    check_against_fp64(host(Cd), A, B, label=f"ragged {entry}")


def _full24(g, shape):
    m = g.integers(1 << 23, 1 << 24, size=shape) | 1
    s = np.where(g.integers(0, 2, size=shape) == 1, -1.0, 1.0)
    return (s * np.ldexp(m.astype(np.float64), g.integers(-20, 20, size=shape) - 23)).astype(np.float32)


@pytest.mark.parametrize("entry", ["fused", "presplit", "presplit_t"])
def test_identity_and_scaled_permutation_exact(fe, entry):
    g = _rng(7)
    n = 160
    X = _full24(g, (n, n))
    I = np.eye(n, dtype=np.float32)
    assert np.array_equal(run(fe, I, X, entry=entry).view(np.uint32), X.view(np.uint32))
    assert np.array_equal(run(fe, X, I, entry=entry).view(np.uint32), X.view(np.uint32))
    P = np.eye(n, dtype=np.float32)[g.permutation(n)]
    D = np.diag(np.ldexp(1.0, g.integers(-10, 10, size=n))).astype(np.float32)
    A = P @ D
    want = (A.astype(np.float64) @ X.astype(np.float64)).astype(np.float32)
    assert np.array_equal(run(fe, A, X, entry=entry), want)


def test_smallest_band_first_case(fe):
    """Bands S0 = 1 + 2^-7 + 2^-16, S1 = 2^-7 + 2^-16, S2 = 2^-8 (exact): the
    smallest-first recombination gives 1 + 2^-7 + 2^-15 + 2^-16 + 2^-23."""
    a = np.array([[1.0, 2.0 ** -16 + 2.0 ** -24, 2.0 ** -7 + 2.0 ** -15 + 2.0 ** -24]], np.float32)
    b = np.ones((3, 1), np.float32)
    C = run(fe, a, b)
    assert C[0, 0] == np.float32(1.0 + 2.0 ** -7 + 2.0 ** -15 + 2.0 ** -16 + 2.0 ** -23)


@pytest.mark.parametrize("lo,hi,emax,K", [(1 << 15, 1 << 16, 0, 64), (1 << 11, 1 << 12, 2, 16),
                                          (1 << 9, 1 << 13, 1, 16), (1 << 19, 1 << 20, 0, 4),
                                          (1 << 23, 1 << 24, 0, 2), (1 << 23, 1 << 24, 2, 5)])
@pytest.mark.parametrize("nbands", [5, 4, 3, 2, 1])
@pytest.mark.parametrize("entry", ["fused", "presplit_t"])
def test_exact_class_bitwise_vs_oracle(fe, orc, lo, hi, emax, K, nbands, entry):
    """On elements whose band sums are exact in any order, GPU == oracle emulation."""
    g = _rng(lo + K + emax)
    M, N = 40, 36

    def draw(shape):
        m = g.integers(lo, hi, size=shape).astype(np.float64)
        m *= np.where(g.integers(0, 2, size=shape) == 1, -1.0, 1.0)
        return np.ldexp(m, g.integers(-emax, emax + 1, size=shape)).astype(np.float32)

    A, B = draw((M, K)), draw((K, N))
    mask = exact_class_mask(A, B)
    assert mask.mean() > 0.3
    C = run(fe, A, B, nbands, entry)
    E = orc.gemm_emu(A, B, nbands)
    assert np.array_equal(C.view(np.uint32)[mask], E.view(np.uint32)[mask])


@pytest.mark.parametrize("nbands,bound", [(1, 2.0 ** -6 + 2.0 ** -13 + 2.0 ** -21 + 2.0 ** -30),
                                          (2, 2.0 ** -13 + 2.0 ** -21 + 2.0 ** -30),
                                          (3, 2.0 ** -21 + 2.0 ** -30), (4, 2.0 ** -30)])
def test_band_drop_ablation(fe, orc, nbands, bound):
    """Keeping bands s < nbands: within bound_b G of the FP64 product and within
    the accumulation bound of the oracle's FP64 truncated-band value."""
    g = _rng(40 + nbands)
    M, N, K = 96, 80, 300
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, nbands).astype(np.float64)
    ref, G = orc.gemm_f64(A, B)
    T = orc.gemm_trunc_f64(A, B, nbands)
    U = 2.0 ** -24
    assert np.all(np.abs(C - T) <= 2 * K * U * G)
    assert np.all(np.abs(C - ref) <= (bound + 2 * K * U) * G)


def test_special_values_class(fe, orc):
    """Inf / NaN inputs: the class of each output (NaN, +Inf, -Inf, finite)
    matches the oracle emulation's class."""
    g = _rng(9)
    M, N, K = 48, 40, 70
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    B[3, :] = np.float32(np.pi)
    A[2, 3] = np.inf
    A[5, 3] = -np.inf
    A[7, 9] = np.nan
    A[11, 3] = np.inf
    B[3, 4] = 1.0                         # Inf * 1.0 meets a zero component -> NaN
    B[20, 30] = np.inf
    A[13, 20] = 0.0                       # Inf * 0 -> NaN in row 13, column 30
    C = run(fe, A, B)
    E = orc.gemm_emu(A, B)

    def cls(X):
        return np.where(np.isnan(X), 0, np.where(X == np.inf, 1, np.where(X == -np.inf, 2, 3)))
    assert np.array_equal(cls(C), cls(E))
    fin = np.isfinite(E)
    assert np.allclose(C[fin], E[fin], rtol=1e-5, atol=1e-5)


def test_subnormals_and_zeros(fe):
    g = _rng(10)
    M, N, K = 64, 64, 64
    A = (g.standard_normal((M, K)) * 2.0 ** -130).astype(np.float32)   # mostly subnormal
    B = g.standard_normal((K, N)).astype(np.float32) * np.float32(2.0 ** 10)
    C = run(fe, A, B)
    check_against_fp64(C, A, B, label="subnormal A", normwise=False)
    Z = np.zeros((M, K), np.float32)
    Z[0, 0] = -0.0
    assert np.all(run(fe, Z, B) == 0)


def test_k_zero_sets_c_to_zero(fe):
    Cd = torch.full((5 * 7,), 3.0, device="cuda")
    fe.sgemm_bf16x9(5, 7, 0, None, 1, None, 7, Cd, 7)
    assert np.all(host(Cd) == 0)


def test_m_or_n_zero_is_noop(fe):
    fe.sgemm_bf16x9(0, 7, 3, None, 3, None, 7, None, 7)
    fe.sgemm_bf16x9(4, 0, 3, None, 3, None, 1, None, 1)


def test_deterministic_bitwise(fe):
    g = _rng(12)
    A = g.standard_normal((513, 700)).astype(np.float32)
    B = g.standard_normal((700, 390)).astype(np.float32)
    c1 = run(fe, A, B)
    c2 = run(fe, A, B)
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))


def test_error_status_raises(fe):
    with pytest.raises(fe.SgemmEmuError):
        fe.sgemm_emu(4, 4, 4, 16, 4, 16, 4, 16, 4, 9)


def test_matmul_helpers(fe):
    g = _rng(13)
    A = torch.from_numpy(g.standard_normal((90, 60)).astype(np.float32)).cuda()
    B = torch.from_numpy(g.standard_normal((60, 70)).astype(np.float32)).cuda()
    C = fe.matmul(A, B)
    Cp = fe.matmul_presplit(A, fe.split(B))
    torch.cuda.synchronize()
    assert torch.equal(C, Cp)
    check_against_fp64(C.cpu().numpy(), A.cpu().numpy(), B.cpu().numpy(), label="matmul")



# ---------------------------------------------------------------- round-to-nearest split (ablation)

def _run_ex(fe, A, B, nbands, flags):
    M, K = A.shape
    N = B.shape[1]
    print(f"gemm ex M={M} N={N} K={K} nbands={nbands} flags={flags}", flush=True, file=sys.stderr)
    Cd = torch.empty((M, N), dtype=torch.float32, device="cuda")
    fe.sgemm_emu_ex(M, N, K, dev(A), K, dev(B), N, Cd, N, nbands, flags)
    return host(Cd)


RNE_SHAPES = [(200, 150, 70), (300, 257, 128), (1100, 260, 256), (1024, 1024, 1024)]


@pytest.mark.parametrize("shape", RNE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_rne_split_gemm_within_bound(fe, orc, shape):
    """SGEMM_EMU_SPLIT_RNE through the in-kernel split (fallback kernel) and the
    workspace split (plane kernel, split-K for the square case): within the
    FP64 bound with nine products, and every band count within the accumulation
    bound of the oracle's truncated-band value under the same split."""
    M, N, K = shape
    g = _rng(M + 2 * N + 3 * K)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    rows = np.sort(g.choice(M, size=min(M, 64), replace=False))
    C = _run_ex(fe, A, B, 5, fe.SGEMM_EMU_SPLIT_RNE)
    check_against_fp64(C[rows], A, B, rows=rows, label=f"rne {shape}")
    _, G = orc.gemm_f64(A, B, rows=rows)
    for nb in (1, 2, 3, 4):
        Cb = _run_ex(fe, A, B, nb, fe.SGEMM_EMU_SPLIT_RNE)[rows].astype(np.float64)
        T = orc.gemm_trunc_f64(A, B, nb, rows=rows, flags=orc.ORC_SPLIT_RNE)
        assert np.all(np.abs(Cb - T) <= 2 * K * 2.0 ** -24 * G), f"nbands={nb}"
    if M >= 1024:
        # the RNE split of B into workspace planes (transposing split kernel)
        W = _run_ex(fe, A, B, 5, fe.SGEMM_EMU_SPLIT_RNE | fe.SGEMM_EMU_PRESPLIT_B)
        if fe.sgemm_emu_split_k(M, N, K) == 1:
            assert np.array_equal(W.view(np.uint32), C.view(np.uint32))
        else:
            check_against_fp64(W[rows], A, B, rows=rows, label=f"rne workspace {shape}")


def test_rne_split_identity_exact_and_smaller_ablation_error(fe, orc):
    g = _rng(71)
    X = (g.standard_normal((64, 64)) * 2.0 ** g.integers(-20, 20, (64, 64))).astype(np.float32)
    I = np.eye(64, dtype=np.float32)
    assert np.array_equal(_run_ex(fe, I, X, 5, fe.SGEMM_EMU_SPLIT_RNE).view(np.uint32), X.view(np.uint32))
    A = g.standard_normal((256, 512)).astype(np.float32)
    B = g.standard_normal((512, 256)).astype(np.float32)
    ref, _ = orc.gemm_f64(A, B)
    e_rz = _run_ex(fe, A, B, 2, 0).astype(np.float64) - ref
    e_rne = _run_ex(fe, A, B, 2, fe.SGEMM_EMU_SPLIT_RNE).astype(np.float64) - ref
    assert np.sqrt(np.mean(e_rne ** 2)) < 0.5 * np.sqrt(np.mean(e_rz ** 2))


# ---------------------------------------------------------------- IEEE fix-up of non-finite inputs

@pytest.mark.parametrize("extra", [0, 8, 16], ids=["default", "presplit", "presplit_a"])
@pytest.mark.parametrize("shape", [(48, 40, 70), (1030, 300, 128), (200, 140, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ieee_specials_fixup(fe, orc, shape, extra):
    """SGEMM_EMU_IEEE_SPECIALS: outputs whose row of A or column of B holds an Inf
    or NaN equal the oracle's plain FP32 dot product bit for bit (+-Inf where the
    emulation gives NaN); all other outputs equal the emulation's.  `extra` = 8
    (SGEMM_EMU_PRESPLIT_B) runs both through the workspace planes where M allows,
    16 (SGEMM_EMU_PRESPLIT_A) also A's planes where K allows."""
    assert extra in (0, fe.SGEMM_EMU_PRESPLIT_B, fe.SGEMM_EMU_PRESPLIT_A)
    M, N, K = shape
    g = _rng(M + N + K + 5)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    B[3, :] = 1.0                          # components (1, 0, 0): Inf x 0 inside the emulation
    A[2, 3] = np.inf                       # row 2: IEEE gives +-Inf, the emulation NaN
    A[5, 3] = -np.inf
    A[7, 9] = np.nan
    B[10, N - 1] = np.inf                  # last column flagged
    B[11, N // 2] = -np.inf
    A[M - 1, 0] = np.nan                   # last row flagged
    C_emu = _run_ex(fe, A, B, 5, extra)
    C = _run_ex(fe, A, B, 5, fe.SGEMM_EMU_IEEE_SPECIALS | extra)
    rows = np.unique([2, 5, 7, M - 1])
    cols = np.unique([N - 1, N // 2])
    flagged = np.zeros((M, N), bool)
    flagged[rows, :] = True
    flagged[:, cols] = True
    naive = orc.sgemm_naive_f32(A, B)
    assert np.array_equal(C[flagged].view(np.uint32), naive[flagged].view(np.uint32))
    assert np.array_equal(C[~flagged].view(np.uint32), C_emu[~flagged].view(np.uint32))
    assert np.isinf(C[2, 0]) and np.isnan(C_emu[2, 0])      # the case the fix-up exists for
    assert np.all(~np.isfinite(C[flagged]))


def test_ieee_specials_fixup_finite_inputs_unchanged(fe):
    g = _rng(99)
    A = g.standard_normal((300, 200)).astype(np.float32)
    B = g.standard_normal((200, 150)).astype(np.float32)
    assert np.array_equal(_run_ex(fe, A, B, 5, fe.SGEMM_EMU_IEEE_SPECIALS).view(np.uint32),
                          _run_ex(fe, A, B, 5, 0).view(np.uint32))


@pytest.mark.parametrize("shape", [(2048, 2048, 2048), (6144, 1024, 256)], ids=lambda s: "x".join(map(str, s)))
def test_presplit_rule_is_invisible(fe, shape):
    """sgemm_bf16x9 splits FP32 B into workspace planes only where that is faster
    (2048^3: yes; 6144x1024x256: no).  Either way the result equals, bit for bit,
    the forced workspace path and the in-kernel split (row blocks below the
    workspace threshold)."""
    M, N, K = shape
    g = _rng(M + N + K + 5)
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    C = run(fe, A, B, entry="fused")
    rows = np.sort(g.choice(M, size=32, replace=False))
    check_against_fp64(C[rows], A, B, rows=rows, label=f"pre-split rule {shape}")
    assert np.array_equal(C.view(np.uint32), run(fe, A, B, entry="fused_ws").view(np.uint32))
    assert np.array_equal(C.view(np.uint32), _fused_in_row_blocks(fe, A, B, 5).view(np.uint32))
