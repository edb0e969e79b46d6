"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid arguments before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm_emu.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    import fp32_emulated_gemm_amd as fe
    return fe.lib()


def test_header_declares_expected_functions():
    import fp32_emulated_gemm_amd as fe
    assert _declared_functions() == sorted(fe.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_serial_lds_debug_library_exports_the_same_symbols():
    """The debug build (one LDS buffer, extra barriers) is built beside the
    library and exports the same C ABI; it reports itself in its version."""
    if os.environ.get("SGEMM_EMU_LIB_OVERRIDE"):
        pytest.skip("a substituted library build is under test")
    import fp32_emulated_gemm_amd as fe
    path = os.path.join(os.path.dirname(os.path.abspath(fe.__file__)), "libsgemm_emu_serial_lds.so")
    D = ctypes.CDLL(path)
    for name in _declared_functions():
        assert hasattr(D, name), name
    D.sgemm_emu_version.restype = ctypes.c_char_p
    assert b"serial-LDS debug build" in D.sgemm_emu_version()


def test_single_hip_runtime_loaded(L):
    import fp32_emulated_gemm_amd as fe
    assert len(fe.hip_runtimes_loaded()) == 1, fe.hip_runtimes_loaded()


def test_products_and_strings(L):
    import fp32_emulated_gemm_amd as fe
    assert [fe.sgemm_emu_products(b) for b in range(0, 7)] == [-1, 1, 3, 6, 8, 9, -1]
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert fe.sgemm_emu_strerror(s) != "unknown status"
    assert fe.sgemm_emu_strerror(7) == "unknown status"
    assert "gfx950" in fe.sgemm_emu_version()


P = 0x10000  # any nonzero, 16-byte aligned address: never dereferenced on these paths


@pytest.mark.parametrize("args,status", [
    ((-1, 4, 4, P, 4, P, 4, P, 4), -1),          # negative M
    ((4, -1, 4, P, 4, P, 4, P, 4), -1),          # negative N
    ((4, 4, -1, P, 4, P, 4, P, 4), -1),          # negative K
    ((4, 4, 8, P, 7, P, 4, P, 4), -1),           # lda < K
    ((4, 8, 4, P, 4, P, 7, P, 8), -1),           # ldb < N
    ((4, 8, 4, P, 4, P, 8, P, 7), -1),           # ldc < N
    ((4, 4, 4, 0, 4, P, 4, P, 4), -2),           # null A
    ((4, 4, 4, P, 4, 0, 4, P, 4), -2),           # null B
    ((4, 4, 4, P, 4, P, 4, 0, 4), -2),           # null C
    ((4, 4, 4, P + 2, 4, P, 4, P, 4), -1),       # misaligned float pointer
    ((1 << 40, 1 << 40, 4, P, 4, P, 1 << 40, P, 1 << 40), -1),  # byte offsets overflow
    ((0, 4, 4, 0, 4, 0, 4, 0, 4), 0),            # empty: no-op, no device needed
    ((4, 0, 4, 0, 4, 0, 1, 0, 1), 0),
])
def test_sgemm_validation_before_any_hip_call(L, args, status):
    assert L.sgemm_bf16x9(*args, None) == status
    assert L.sgemm_emu(*args, 5, None) == status


@pytest.mark.parametrize("nbands", [0, 6, -3])
def test_bad_nbands(L, nbands):
    assert L.sgemm_emu(4, 4, 4, P, 4, P, 4, P, 4, nbands, None) == -1
    assert L.sgemm_emu_presplit_b(4, 4, 4, P, 4, P, P, P, 4, 0, P, 4, nbands, None) == -1
    assert L.sgemm_emu_split_k(4, 4, 4, nbands) == -1
    assert L.sgemm_emu_split_k_fp32_b(4, 4, 4, nbands) == -1


def test_presplit_validation(L):
    assert L.sgemm_emu_presplit_b(4, 4, 4, P, 4, P, 0, P, 4, 0, P, 4, 5, None) == -2
    assert L.sgemm_emu_presplit_b(4, 4, 4, P, 4, P + 1, P, P, 4, 0, P, 4, 5, None) == -1
    assert L.sgemm_emu_presplit_b(4, 8, 4, P, 4, P, P, P, 7, 0, P, 8, 5, None) == -1   # K x N: ldb < N
    assert L.sgemm_emu_presplit_b(4, 8, 6, P, 6, P, P, P, 5, 1, P, 8, 5, None) == -1   # N x K: ldb < K
    assert L.sgemm_emu_presplit_b(4, 8, 4, P, 4, P, P, P, 8, 2, P, 8, 5, None) == -1   # unknown layout


def test_linear_validation(L):
    # sgemm_emu_linear(M, N, K, X, ldx, W0, W1, W2, ldw, bias, act, Y, ldy, nbands, stream); W is N x K
    assert L.sgemm_emu_linear(4, 8, 6, P, 6, P, P, P, 5, None, 0, P, 8, 5, None) == -1    # ldw < K
    assert L.sgemm_emu_linear(4, 8, 6, P, 6, P, P, 0, 6, None, 0, P, 8, 5, None) == -2    # null plane
    assert L.sgemm_emu_linear(4, 8, 6, P, 6, P, P, P, 6, P + 2, 0, P, 8, 5, None) == -1   # misaligned bias
    assert L.sgemm_emu_linear(4, 8, 6, P, 6, P, P, P, 6, None, 0, P, 7, 5, None) == -1    # ldy < N
    assert L.sgemm_emu_linear(4, 8, 6, P, 6, P, P, P, 6, P, 0, P, 8, 0, None) == -1       # nbands
    assert L.sgemm_emu_linear(0, 8, 6, 0, 6, P, P, P, 6, P, 0, 0, 8, 5, None) == 0        # empty
    assert L.sgemm_emu_linear(4, 8, 6, P, 6, P, P, P, 6, P, 2, P, 8, 5, None) == -1       # activation
    assert L.sgemm_emu_linear(4, 8, 6, P, 6, P, P, P, 6, P, -1, P, 8, 5, None) == -1
    import torch
    if not torch.cuda.is_available():
        assert L.sgemm_emu_linear(4, 8, 6, P, 6, P, P, P, 6, P, 0, P, 8, 5, None) == -3


def test_split_validation(L):
    assert L.split_f32_bf16x3(-1, 4, P, 4, P, P, P, 4, None) == -1
    assert L.split_f32_bf16x3(4, 4, P, 3, P, P, P, 4, None) == -1
    assert L.split_f32_bf16x3(4, 4, P, 4, P, P, P, 3, None) == -1
    assert L.split_f32_bf16x3(4, 4, 0, 4, P, P, P, 4, None) == -2
    assert L.split_f32_bf16x3(0, 4, 0, 4, 0, 0, 0, 4, None) == 0


def test_ex_entry_flags(L):
    assert L.sgemm_emu_ex(4, 4, 4, P, 4, P, 4, P, 4, 5, 2, None) == -1     # transpose is a split flag
    assert L.sgemm_emu_ex(4, 4, 4, P, 4, P, 4, P, 4, 5, 256, None) == -1   # unknown flag
    assert L.sgemm_emu_ex(4, 4, 4, P, 4, P, 4, P, 4, 5, 128 | 8, None) == -1   # no workspace and pre-split
    assert L.sgemm_emu_ex(4, 4, 4, P, 4, P, 4, P, 4, 5, 128 | 32, None) == -1  # no workspace and a strategy
    assert L.sgemm_emu_ex(4, 4, 4, P, 4, P, 4, P, 4, 5, 128 | 4, None) == -1   # no workspace and IEEE fix-up
    assert L.sgemm_emu_ex(0, 4, 4, 0, 4, 0, 4, 0, 4, 5, 128 | 1, None) == 0    # no workspace, RNE: empty
    assert L.sgemm_emu_ex(4, 4, 4, P, 4, P, 4, P, 4, 4, 32, None) == -1    # performant needs nbands 5
    assert L.sgemm_emu_ex(4, 4, 4, P, 4, P, 4, P, 4, 5, 64 | 1, None) == -1  # native: no RNE split
    assert L.sgemm_emu_ex(4, 4, 4, P, 3, P, 4, P, 4, 5, 64, None) == -1    # native: lda < K
    assert L.sgemm_emu_ex(0, 4, 4, 0, 4, 0, 4, 0, 4, 5, 32, None) == 0     # performant: empty
    assert L.sgemm_emu_ex(0, 4, 4, 0, 4, 0, 4, 0, 4, 5, 8 | 1, None) == 0  # pre-split B flag: empty
    assert L.sgemm_emu_ex(0, 4, 4, 0, 4, 0, 4, 0, 4, 5, 16 | 1, None) == 0  # pre-split A flag: empty
    assert L.sgemm_emu_ex(4, 4, 4, P, 4, P, 4, P, 4, 0, 1, None) == -1     # nbands
    assert L.sgemm_emu_ex(0, 4, 4, 0, 4, 0, 4, 0, 4, 5, 1, None) == 0      # empty
    assert L.split_f32_bf16x3_ex(4, 4, P, 4, P, P, P, 4, 4, None) == -1    # unknown flag
    assert L.split_f32_bf16x3_ex(6, 4, P, 4, P, P, P, 5, 2, None) == -1    # transposed: ldo < rows
    assert L.split_f32_bf16x3_ex(6, 4, P, 4, P, P, P, 3, 1, None) == -1    # plain: ldo < cols
    assert L.split_f32_bf16x3_ex(0, 4, 0, 4, 0, 0, 0, 4, 3, None) == 0


def test_split_transposed_validation(L):
    # X is rows x cols (ldx >= cols); the planes are cols x rows (ldo >= rows)
    assert L.split_f32_bf16x3_transposed(-1, 4, P, 4, P, P, P, 4, None) == -1
    assert L.split_f32_bf16x3_transposed(6, 4, P, 3, P, P, P, 6, None) == -1
    assert L.split_f32_bf16x3_transposed(6, 4, P, 4, P, P, P, 5, None) == -1
    assert L.split_f32_bf16x3_transposed(6, 4, P, 4, P, 0, P, 6, None) == -2
    assert L.split_f32_bf16x3_transposed(0, 4, 0, 4, 0, 0, 0, 1, None) == 0


def test_valid_call_without_gpu_reports_arch(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert L.sgemm_bf16x9(4, 4, 4, P, 4, P, 4, P, 4, None) == -3
    assert L.split_f32_bf16x3(4, 4, P, 4, P, P, P, 4, None) == -3
    assert L.sgemm_emu_release_workspace() == -3
    assert L.sgemm_emu_split_k_fp32_b(1024, 1024, 1024, 5) == -3
    assert L.sgemm_emu_split_k_fp32_b(-1, 4, 4, 5) == -1


def test_leading_dimension_limit(L):
    """lda / ldb up to 8,388,544 elements (a 128-row tile span in 32-bit byte
    offsets); one more is rejected before any HIP call."""
    top = (1 << 32) // (128 * 4) - 64
    assert L.sgemm_bf16x9(4, 4, 4, P, top + 1, P, 4, P, 4, None) == -1
    assert L.sgemm_bf16x9(4, 4, 4, P, 4, P, top + 1, P, 4, None) == -1
    assert L.sgemm_emu_presplit_b(4, 4, 4, P, 4, P, P, P, top + 1, 1, P, 4, 5, None) == -1
    # the C stores of a 128-row tile use 32-bit offsets too: ldc and the linear
    # layer's ldy have the same limit
    assert L.sgemm_bf16x9(4, 4, 4, P, 4, P, 4, P, top + 1, None) == -1
    assert L.sgemm_emu(4, 4, 4, P, 4, P, 4, P, top + 1, 5, None) == -1
    assert L.sgemm_emu_presplit_b(4, 4, 4, P, 4, P, P, P, 4, 1, P, top + 1, 5, None) == -1
    assert L.sgemm_emu_linear(4, 4, 4, P, 4, P, P, P, 4, None, 0, P, top + 1, 5, None) == -1


def test_tensor_wrappers_reject_bad_tensors():
    """The tensor conveniences check dtype, layout and device before the
    library sees a pointer (a wrong tensor would otherwise be read out of
    bounds on the GPU)."""
    import torch
    import fp32_emulated_gemm_amd as fe
    a = torch.zeros((8, 8), dtype=torch.float32)
    with pytest.raises(TypeError):
        fe.matmul(a.half(), a)                                  # float16 would be read at twice its size
    with pytest.raises(TypeError):
        fe.split(a.double())
    with pytest.raises(ValueError):
        fe.matmul(torch.zeros(8, dtype=torch.float32).expand(8, 8), a)   # broadcast rows overlap
    with pytest.raises(ValueError):
        fe.matmul(a.t(), a)                                     # column stride != 1
    with pytest.raises(ValueError):
        fe.split_t(torch.zeros((2, 4, 4)))                      # not 2-D
    with pytest.raises(ValueError):
        fe.matmul(a, a)                                         # host memory
    planes = [torch.zeros((8, 8), dtype=torch.int16) for _ in range(3)]
    with pytest.raises(TypeError):
        fe.matmul_presplit(a, [planes[0], planes[1], planes[2].float()])
    with pytest.raises(ValueError):
        fe.matmul_presplit(a, [planes[0], planes[1], torch.zeros((8, 9), dtype=torch.int16)[:, :8]])
    with pytest.raises(ValueError):
        fe.matmul_presplit(a, planes[:2])
