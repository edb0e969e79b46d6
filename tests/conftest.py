"""Shared test set-up: the `gpu` marker, import paths and small helpers."""
import ctypes
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


_PINS = None


def pins_lib():
    """Build (once per session) and load the C property checkers in tests/native."""
    global _PINS
    if _PINS is None:
        src = os.path.join(ROOT, "tests", "native", "pins.c")
        out = os.environ.get("PINS_LIB_OVERRIDE") or os.path.join(ROOT, "tests", "native", "libpins.so")
        if "PINS_LIB_OVERRIDE" in os.environ:
            pass              # a prebuilt copy (the sanitizer run builds its own)
        elif not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
            subprocess.run(["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off",
                            "-fopenmp", "-fPIC", "-shared", "-o", out + ".tmp", src, "-lm"],
                           check=True)
            os.replace(out + ".tmp", out)
        L = ctypes.CDLL(out)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.pin_split_range.argtypes = [ctypes.c_uint64, i64, vp, vp, vp, ctypes.POINTER(ctypes.c_uint64)]
        L.pin_split_range.restype = i64
        L.pin_split_rne_range.argtypes = [ctypes.c_uint64, i64, vp, vp, vp, ctypes.POINTER(ctypes.c_uint64)]
        L.pin_split_rne_range.restype = i64
        L.pin_bf16_products.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(i64)]
        L.pin_bf16_products.restype = i64
        L.pin_band_algebra.argtypes = [i64] + [vp] * 8
        L.pin_band_algebra.restype = i64
        _PINS = L
    return _PINS


@pytest.fixture(scope="session")
def pins():
    return pins_lib()


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
