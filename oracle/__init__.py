"""CPU oracle for the BF16x9 emulated FP32 GEMM -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never calls it, and nothing here imports
the GPU library: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, built by ``oracle/build.py``);
this module only marshals numpy arrays into it.  Every function follows the
pages cited in ``oracle.c``:

  [NVB] NVIDIA Technical Blog, "Unlocking Tensor Core Performance for Machine
        Learning Interatomic Potentials" (2026-10-29).
  [KR]  discuss.pytorch.kr summary of the same post.

Functions:
  split(X, mode)          -> (X0, X1, X2) uint16 BF16 bit patterns
                             ([KR] "Blackwell의 BF16x9", x = x0 + 2^-8 x1 + 2^-16 x2);
                             mode SPLIT_RZ (the method's reading) or SPLIT_RNE (ablation)
  gemm_f64(A, B, rows)    -> (Cref, G) FP64 reference and sum |a*b|
  sgemm_naive_f32(A, B)   -> C, sequential FP32 accumulation (CPU baseline)
  gemm_emu(A, B, nbands)  -> C, scalar band emulation ([NVB] Fig. 1 caption)
  gemm_trunc_f64(A, B, b) -> T_b, the FP64 value of the kept products
  gelu_f64_to_f32(x)      -> fp32(x Phi(x)), exact GELU (erfc form) in double
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

ORC_SPLIT_RNE = 2            # gemm_emu / gemm_trunc_f64 flag: round-to-nearest split
SPLIT_RZ, SPLIT_RNE = 0, 1   # split modes

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def lib():
    """Load liboracle.so, building it first if it is missing or stale."""
    global _LIB
    if _LIB is None:
        # A test may point this at a deliberately broken copy of the oracle to
        # show that the pins catch the planted mistake.
        path = os.environ.get("ORACLE_LIB_OVERRIDE") or _build.build(force=False)
        L = ctypes.CDLL(path)
        L.orc_split_one.argtypes = [ctypes.c_float, ctypes.POINTER(ctypes.c_uint16),
                                    ctypes.POINTER(ctypes.c_uint16), ctypes.POINTER(ctypes.c_uint16)]
        L.orc_split_one.restype = None
        L.orc_split.argtypes = [_i64, _i64, _vp, _i64, _vp, _vp, _vp, _i64]
        L.orc_split_mode.argtypes = [_i64, _i64, _vp, _i64, _vp, _vp, _vp, _i64, ctypes.c_int]
        L.orc_split_one_mode.argtypes = [ctypes.c_float, ctypes.c_int, ctypes.POINTER(ctypes.c_uint16),
                                         ctypes.POINTER(ctypes.c_uint16), ctypes.POINTER(ctypes.c_uint16)]
        L.orc_split_one_mode.restype = None
        L.orc_gemm_f64.argtypes = [_i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64]
        L.orc_sgemm_naive_f32.argtypes = [_i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64]
        L.orc_gemm_emu.argtypes = [_i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                   ctypes.c_int, ctypes.c_int, _vp]
        L.orc_gemm_trunc_f64.argtypes = [_i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                         ctypes.c_int, ctypes.c_int]
        L.orc_gelu_f64_to_f32.argtypes = [_i64, _vp, _vp]
        L.orc_num_threads.argtypes = []
        for name in ("orc_split", "orc_split_mode", "orc_gemm_f64", "orc_sgemm_naive_f32", "orc_gemm_emu",
                     "orc_gemm_trunc_f64", "orc_gelu_f64_to_f32", "orc_num_threads"):
            getattr(L, name).restype = ctypes.c_int
        _LIB = L
    return _LIB


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"oracle {name} failed with status {rc}")


def _mat(a, dtype=np.float32):
    a = np.ascontiguousarray(a, dtype=dtype)
    if a.ndim != 2:
        raise ValueError("expected a 2-D array")
    return a


def _rows(rows, M):
    if rows is None:
        return None, M
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.ndim != 1 or (r.size and (r.min() < 0 or r.max() >= M)):
        raise ValueError("row indices out of range")
    return r, r.size


def num_threads() -> int:
    """OpenMP threads the oracle uses (all host cores unless OMP_NUM_THREADS says otherwise)."""
    return lib().orc_num_threads()


def split_one(x: float, mode=SPLIT_RZ):
    """Split one FP32 value; returns the three BF16 bit patterns (x0, x1, x2)."""
    c = [ctypes.c_uint16() for _ in range(3)]
    if mode == SPLIT_RZ:
        lib().orc_split_one(ctypes.c_float(x), *[ctypes.byref(v) for v in c])
    else:
        lib().orc_split_one_mode(ctypes.c_float(x), int(mode), *[ctypes.byref(v) for v in c])
    return tuple(v.value for v in c)


def split(X, mode=SPLIT_RZ):
    """Elementwise split of a float32 array of any shape into three uint16 arrays."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    flat = X.reshape(1, -1) if X.size else X.reshape(0, 0)
    outs = [np.empty(flat.shape, dtype=np.uint16) for _ in range(3)]
    if flat.size:
        _check(lib().orc_split_mode(flat.shape[0], flat.shape[1], _ptr(flat), flat.shape[1],
                                    *[_ptr(o) for o in outs], flat.shape[1], int(mode)), "split")
    return tuple(o.reshape(X.shape) for o in outs)


def gemm_f64(A, B, rows=None, want_g=True):
    """FP64 reference C = A B (k ascending) and G = sum_k |a b|; optionally only `rows` of A."""
    A, B = _mat(A), _mat(B)
    M, K = A.shape
    if B.shape[0] != K:
        raise ValueError("inner dimensions differ")
    N = B.shape[1]
    r, nr = _rows(rows, M)
    C = np.empty((nr, N), dtype=np.float64)
    G = np.empty((nr, N), dtype=np.float64) if want_g else None
    _check(lib().orc_gemm_f64(nr, _ptr(r), N, K, _ptr(A), max(K, 1), _ptr(B), max(N, 1),
                              _ptr(C), max(N, 1), _ptr(G), max(N, 1)), "gemm_f64")
    return (C, G) if want_g else C


def sgemm_naive_f32(A, B, rows=None):
    """Naive FP32 SGEMM: sequential FP32 accumulator, product and sum rounded separately."""
    A, B = _mat(A), _mat(B)
    M, K = A.shape
    if B.shape[0] != K:
        raise ValueError("inner dimensions differ")
    N = B.shape[1]
    r, nr = _rows(rows, M)
    C = np.empty((nr, N), dtype=np.float32)
    _check(lib().orc_sgemm_naive_f32(nr, _ptr(r), N, K, _ptr(A), max(K, 1), _ptr(B), max(N, 1),
                                     _ptr(C), max(N, 1)), "sgemm_naive_f32")
    return C


def gemm_emu(A, B, nbands=5, rows=None, flags=0, want_bands=False):
    """Scalar band emulation of the BF16x9 GEMM; keeps bands s < nbands."""
    A, B = _mat(A), _mat(B)
    M, K = A.shape
    if B.shape[0] != K:
        raise ValueError("inner dimensions differ")
    N = B.shape[1]
    r, nr = _rows(rows, M)
    C = np.empty((nr, N), dtype=np.float32)
    S = np.empty((5, nr, N), dtype=np.float32) if want_bands else None
    _check(lib().orc_gemm_emu(nr, _ptr(r), N, K, _ptr(A), max(K, 1), _ptr(B), max(N, 1),
                              _ptr(C), max(N, 1), int(nbands), int(flags), _ptr(S)), "gemm_emu")
    return (C, S) if want_bands else C


def gemm_trunc_f64(A, B, nbands=5, rows=None, flags=0):
    """FP64 value of the kept products: sum over p+q < nbands of 2^-8(p+q) A_p B_q."""
    A, B = _mat(A), _mat(B)
    M, K = A.shape
    if B.shape[0] != K:
        raise ValueError("inner dimensions differ")
    N = B.shape[1]
    r, nr = _rows(rows, M)
    T = np.empty((nr, N), dtype=np.float64)
    _check(lib().orc_gemm_trunc_f64(nr, _ptr(r), N, K, _ptr(A), max(K, 1), _ptr(B), max(N, 1),
                                    _ptr(T), max(N, 1), int(nbands), int(flags)), "gemm_trunc_f64")
    return T


def gelu_f64_to_f32(x):
    """fp32(x Phi(x)) = fp32(0.5 x erfc(-x / sqrt 2)), evaluated in double."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, dtype=np.float32)
    if x.size:
        _check(lib().orc_gelu_f64_to_f32(x.size, _ptr(x), _ptr(y)), "gelu")
    return y
