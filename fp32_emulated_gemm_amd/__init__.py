"""Python binding of libsgemm_emu -- FP32 GEMM emulated on MI355X BF16 MFMA (BF16x9).

Thin ctypes marshalling over the C ABI in ``include/sgemm_emu.h``; every step
of the computation runs in the library's HIP kernels.  PyTorch supplies device
memory and streams only.  The functions keep the C names and argument order:

    sgemm_bf16x9(M, N, K, A, lda, B, ldb, C, ldc, stream=None)
    sgemm_emu(M, N, K, A, lda, B, ldb, C, ldc, nbands, stream=None)
    sgemm_emu_ex(M, N, K, A, lda, B, ldb, C, ldc, nbands, flags, stream=None)
    sgemm_emu_presplit_b(M, N, K, A, lda, B0, B1, B2, ldb, b_layout, C, ldc, nbands, stream=None)
    sgemm_emu_presplit_b_noalloc(M, N, K, A, lda, B0, B1, B2, ldb, C, ldc, nbands, stream=None)
    sgemm_emu_linear(M, N, K, X, ldx, W0, W1, W2, ldw, bias, activation, Y, ldy, nbands, stream=None)
    split_f32_bf16x3(rows, cols, X, ldx, X0, X1, X2, ldo, stream=None)
    split_f32_bf16x3_transposed(rows, cols, X, ldx, X0, X1, X2, ldo, stream=None)
    split_f32_bf16x3_ex(rows, cols, X, ldx, X0, X1, X2, ldo, flags, stream=None)
    sgemm_emu_split_k(M, N, K, nbands), sgemm_emu_split_k_fp32_b(M, N, K, nbands)
    sgemm_emu_release_workspace()
    sgemm_emu_products(nbands), sgemm_emu_strerror(status), sgemm_emu_version()

Matrix arguments may be torch tensors (their data pointer is passed; they must
live on the current HIP device) or raw integer device addresses.  `stream`
defaults to torch's current stream.  A nonzero status raises SgemmEmuError.

Convenience wrappers that allocate outputs: ``matmul``, ``matmul_presplit``,
``split``, ``split_t``.  They check their tensors first (dtype, the current HIP
device, 2-D row-major with non-overlapping rows, matching planes) and raise
TypeError / ValueError before the library sees a pointer.

The library links the same HIP runtime soname as PyTorch, so torch is imported
first: the library then binds to the runtime torch already loaded and both see
the same devices, pointers and streams.  If the built library is missing, the
import of the GPU functions fails loudly; there is no fallback.
"""
import ctypes
import os

import torch  # noqa: F401  (must be loaded before the library, see above)

HERE = os.path.dirname(os.path.abspath(__file__))
# SGEMM_EMU_LIB_OVERRIDE: load another build of the library (the test suite's
# host-only sanitizer build); unset, the in-tree build.
LIB_PATH = os.environ.get("SGEMM_EMU_LIB_OVERRIDE") or os.path.join(HERE, "libsgemm_emu.so")

SGEMM_EMU_OK = 0
SGEMM_EMU_EINVAL = -1
SGEMM_EMU_ENULL = -2
SGEMM_EMU_EARCH = -3
SGEMM_EMU_ELAUNCH = -4
SGEMM_EMU_ENOMEM = -5
SGEMM_EMU_ECAPTURE = -6
SGEMM_EMU_B_KN = 0   # pre-split planes K x N (split of B)
SGEMM_EMU_B_NK = 1   # pre-split planes N x K (split of B^T, e.g. a weight stored [out][in])
SGEMM_EMU_ACT_NONE = 0
SGEMM_EMU_ACT_GELU = 1  # GELU, exact (erf) form
SGEMM_EMU_SPLIT_RNE = 1        # flag: round-to-nearest-even split (rounding ablation)
SGEMM_EMU_SPLIT_TRANSPOSE = 2  # flag (split_f32_bf16x3_ex): planes of X^T
SGEMM_EMU_IEEE_SPECIALS = 4    # flag (sgemm_emu_ex): IEEE FP32 results where inputs hold Inf/NaN
SGEMM_EMU_PRESPLIT_B = 8       # flag (sgemm_emu_ex): split FP32 B once into workspace planes whenever allowed
SGEMM_EMU_PRESPLIT_A = 16      # flag (sgemm_emu_ex): split FP32 A (and B) once into workspace planes whenever allowed
SGEMM_EMU_PERFORMANT = 32      # flag (sgemm_emu_ex): emulate only where faster than the native FP32 kernel
SGEMM_EMU_NATIVE_FP32 = 64     # flag (sgemm_emu_ex): the library's native FP32 kernel
SGEMM_EMU_NO_WORKSPACE = 128   # flag (sgemm_emu_ex): in-kernel split, no stream-K, nothing allocated

EXPORTS = ("sgemm_bf16x9", "sgemm_emu", "sgemm_emu_ex", "sgemm_emu_presplit_b", "sgemm_emu_presplit_b_noalloc",
           "sgemm_emu_linear",
           "split_f32_bf16x3", "split_f32_bf16x3_transposed", "split_f32_bf16x3_ex", "sgemm_emu_split_k",
           "sgemm_emu_split_k_fp32_b", "sgemm_emu_release_workspace", "sgemm_emu_products", "sgemm_emu_strerror",
           "sgemm_emu_version")


class SgemmEmuError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({sgemm_emu_strerror(status)})")


_LIB = None


def lib():
    """Load libsgemm_emu.so (built in-tree by fp32_emulated_gemm_amd.build)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m fp32_emulated_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.sgemm_bf16x9.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
        L.sgemm_emu.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, vp]
        L.sgemm_emu_ex.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, ci, vp]
        L.sgemm_emu_presplit_b.argtypes = [i64, i64, i64, vp, i64, vp, vp, vp, i64, ci, vp, i64, ci, vp]
        L.sgemm_emu_presplit_b_noalloc.argtypes = [i64, i64, i64, vp, i64, vp, vp, vp, i64, vp, i64, ci, vp]
        L.sgemm_emu_linear.argtypes = [i64, i64, i64, vp, i64, vp, vp, vp, i64, vp, ci, vp, i64, ci, vp]
        L.split_f32_bf16x3.argtypes = [i64, i64, vp, i64, vp, vp, vp, i64, vp]
        L.split_f32_bf16x3_transposed.argtypes = [i64, i64, vp, i64, vp, vp, vp, i64, vp]
        L.split_f32_bf16x3_ex.argtypes = [i64, i64, vp, i64, vp, vp, vp, i64, ci, vp]
        L.sgemm_emu_split_k.argtypes = [i64, i64, i64, ci]
        L.sgemm_emu_split_k_fp32_b.argtypes = [i64, i64, i64, ci]
        L.sgemm_emu_release_workspace.argtypes = []
        L.sgemm_emu_products.argtypes = [ci]
        L.sgemm_emu_strerror.argtypes = [ci]
        L.sgemm_emu_strerror.restype = ctypes.c_char_p
        L.sgemm_emu_version.argtypes = []
        L.sgemm_emu_version.restype = ctypes.c_char_p
        for n in ("sgemm_bf16x9", "sgemm_emu", "sgemm_emu_ex", "sgemm_emu_presplit_b", "sgemm_emu_presplit_b_noalloc",
                  "sgemm_emu_linear",
                  "split_f32_bf16x3", "split_f32_bf16x3_transposed", "split_f32_bf16x3_ex", "sgemm_emu_split_k",
                  "sgemm_emu_split_k_fp32_b", "sgemm_emu_release_workspace", "sgemm_emu_products"):
            getattr(L, n).restype = ci
        _LIB = L
    return _LIB


def hip_runtimes_loaded():
    """Paths of the HIP runtime libraries mapped into this process (expect one)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            p = line.split()[-1]
            if "libamdhip64.so" in p:
                paths.add(os.path.realpath(p))
    return sorted(paths)


def _addr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr() if x.numel() else (x.data_ptr() or None)
    return int(x)


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    return int(s)


def _ok(status, where):
    if status != SGEMM_EMU_OK:
        raise SgemmEmuError(status, where)
    return status


def sgemm_bf16x9(M, N, K, A, lda, B, ldb, C, ldc, stream=None):
    return _ok(lib().sgemm_bf16x9(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, _stream(stream)),
               "sgemm_bf16x9")


def sgemm_emu(M, N, K, A, lda, B, ldb, C, ldc, nbands, stream=None):
    return _ok(lib().sgemm_emu(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, nbands, _stream(stream)),
               "sgemm_emu")


def sgemm_emu_ex(M, N, K, A, lda, B, ldb, C, ldc, nbands, flags, stream=None):
    return _ok(lib().sgemm_emu_ex(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, nbands, flags,
                                  _stream(stream)), "sgemm_emu_ex")


def sgemm_emu_presplit_b(M, N, K, A, lda, B0, B1, B2, ldb, b_layout, C, ldc, nbands, stream=None):
    return _ok(lib().sgemm_emu_presplit_b(M, N, K, _addr(A), lda, _addr(B0), _addr(B1), _addr(B2), ldb,
                                          b_layout, _addr(C), ldc, nbands, _stream(stream)),
               "sgemm_emu_presplit_b")


def sgemm_emu_presplit_b_noalloc(M, N, K, A, lda, B0, B1, B2, ldb, C, ldc, nbands, stream=None):
    return _ok(lib().sgemm_emu_presplit_b_noalloc(M, N, K, _addr(A), lda, _addr(B0), _addr(B1), _addr(B2), ldb,
                                                  _addr(C), ldc, nbands, _stream(stream)),
               "sgemm_emu_presplit_b_noalloc")


def sgemm_emu_linear(M, N, K, X, ldx, W0, W1, W2, ldw, bias, activation, Y, ldy, nbands, stream=None):
    return _ok(lib().sgemm_emu_linear(M, N, K, _addr(X), ldx, _addr(W0), _addr(W1), _addr(W2), ldw, _addr(bias),
                                      activation, _addr(Y), ldy, nbands, _stream(stream)), "sgemm_emu_linear")


def split_f32_bf16x3(rows, cols, X, ldx, X0, X1, X2, ldo, stream=None):
    return _ok(lib().split_f32_bf16x3(rows, cols, _addr(X), ldx, _addr(X0), _addr(X1), _addr(X2), ldo,
                                      _stream(stream)), "split_f32_bf16x3")


def split_f32_bf16x3_transposed(rows, cols, X, ldx, X0, X1, X2, ldo, stream=None):
    return _ok(lib().split_f32_bf16x3_transposed(rows, cols, _addr(X), ldx, _addr(X0), _addr(X1), _addr(X2), ldo,
                                                 _stream(stream)), "split_f32_bf16x3_transposed")


def split_f32_bf16x3_ex(rows, cols, X, ldx, X0, X1, X2, ldo, flags, stream=None):
    return _ok(lib().split_f32_bf16x3_ex(rows, cols, _addr(X), ldx, _addr(X0), _addr(X1), _addr(X2), ldo, flags,
                                         _stream(stream)), "split_f32_bf16x3_ex")


def sgemm_emu_split_k(M, N, K, nbands=5):
    status = lib().sgemm_emu_split_k(M, N, K, nbands)
    return _ok(status, "sgemm_emu_split_k") if status < 0 else status


def sgemm_emu_split_k_fp32_b(M, N, K, nbands=5):
    status = lib().sgemm_emu_split_k_fp32_b(M, N, K, nbands)
    return _ok(status, "sgemm_emu_split_k_fp32_b") if status < 0 else status


def sgemm_emu_release_workspace():
    return _ok(lib().sgemm_emu_release_workspace(), "sgemm_emu_release_workspace")


def sgemm_emu_products(nbands):
    return lib().sgemm_emu_products(nbands)


def sgemm_emu_strerror(status):
    return lib().sgemm_emu_strerror(status).decode()


def sgemm_emu_version():
    return lib().sgemm_emu_version().decode()


# ---------------------------------------------------------------- tensor conveniences

_PLANE_DTYPES = (torch.int16, torch.bfloat16)
_F32 = (torch.float32,)


def _layout(t, name, dtypes):
    """Leading dimension of t after checking that it is a 2-D row-major tensor of
    one of `dtypes` whose rows do not overlap.  The library reads and writes
    through raw pointers: a tensor that failed these checks would make it touch
    memory the tensor does not own."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: expected dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name}: expected a 2-D tensor, got {t.dim()} dimensions")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: expected unit stride along columns, got {t.stride(1)}")
    if rows > 1 and cols > 0 and t.stride(0) < cols:
        raise ValueError(f"{name}: rows overlap (row stride {t.stride(0)} < {cols} columns)")
    return max(t.stride(0), cols, 1)


def _on_device(*named):
    """Every (name, tensor) must live on the current HIP device."""
    for name, t in named:
        if t.device.type != "cuda":
            raise ValueError(f"{name}: expected a tensor on the current HIP device, got {t.device}")
        if t.device.index != torch.cuda.current_device():
            raise ValueError(f"{name}: expected a tensor on the current HIP device "
                             f"(cuda:{torch.cuda.current_device()}), got {t.device}")


def _ld(t):
    """Leading dimension of a row-major 2-D FP32 tensor on the current device."""
    ld = _layout(t, "tensor", _F32)
    _on_device(("tensor", t))
    return ld


def _planes(parts, name):
    """Layout of three BF16 component planes of one shape and leading dimension."""
    if len(parts) != 3:
        raise ValueError(f"{name}: expected three planes, got {len(parts)}")
    lds = [_layout(p, f"{name}[{i}]", _PLANE_DTYPES) for i, p in enumerate(parts)]
    if any(p.shape != parts[0].shape for p in parts) or len(set(lds)) != 1:
        raise ValueError(f"{name}: the three planes differ in shape or leading dimension")
    return lds[0]


def _out(out, M, N, like):
    """The output tensor (allocated on `like`'s device if None) and its leading dimension."""
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=like.device)
    ld = _layout(out, "out", _F32)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out: expected shape {(M, N)}, got {tuple(out.shape)}")
    return out, ld


def matmul(A, B, nbands=5, out=None, stream=None):
    """C = A @ B for float32 CUDA tensors, through sgemm_emu (nbands=5: sgemm_bf16x9)."""
    lda, ldb = _layout(A, "A", _F32), _layout(B, "B", _F32)
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    _on_device(("A", A), ("B", B))
    C, ldc = _out(out, M, N, A)
    _on_device(("out", C))
    if nbands == 5:
        sgemm_bf16x9(M, N, K, A, lda, B, ldb, C, ldc, stream)
    else:
        sgemm_emu(M, N, K, A, lda, B, ldb, C, ldc, nbands, stream)
    return C


def split(X, stream=None):
    """Three uint16 tensors (BF16 bit patterns, stored as int16) holding X's components."""
    ldx = _layout(X, "X", _F32)
    _on_device(("X", X))
    rows, cols = X.shape
    outs = [torch.empty((rows, cols), dtype=torch.int16, device=X.device) for _ in range(3)]
    split_f32_bf16x3(rows, cols, X, ldx, outs[0], outs[1], outs[2], max(cols, 1), stream)
    return tuple(outs)


def split_t(X, stream=None):
    """The components of X^T (cols x rows) as three int16 tensors, from X directly."""
    ldx = _layout(X, "X", _F32)
    _on_device(("X", X))
    rows, cols = X.shape
    outs = [torch.empty((cols, rows), dtype=torch.int16, device=X.device) for _ in range(3)]
    split_f32_bf16x3_transposed(rows, cols, X, ldx, outs[0], outs[1], outs[2], max(rows, 1), stream)
    return tuple(outs)


def matmul_presplit(A, Bparts, nbands=5, out=None, stream=None, b_layout=SGEMM_EMU_B_KN):
    """C = A @ B with B given as its three component planes (from `split`):
    planes of B (K x N) for SGEMM_EMU_B_KN, planes of B^T (N x K) for SGEMM_EMU_B_NK."""
    lda = _layout(A, "A", _F32)
    ldb = _planes(Bparts, "Bparts")
    M, K = A.shape
    if b_layout == SGEMM_EMU_B_KN:
        K2, N = Bparts[0].shape
    elif b_layout == SGEMM_EMU_B_NK:
        N, K2 = Bparts[0].shape
    else:
        raise ValueError(f"unknown b_layout {b_layout}")
    if K2 != K:
        raise ValueError("inner dimensions differ")
    _on_device(("A", A), *((f"Bparts[{i}]", p) for i, p in enumerate(Bparts)))
    C, ldc = _out(out, M, N, A)
    _on_device(("out", C))
    sgemm_emu_presplit_b(M, N, K, A, lda, Bparts[0], Bparts[1], Bparts[2], ldb, b_layout, C, ldc,
                         nbands, stream)
    return C
