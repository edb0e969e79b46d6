"""The CPU-side code under AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (oracle/oracle.c) and the property checkers (tests/native/pins.c)
  are rebuilt with gcc's -fsanitize=address,undefined and the oracle's pin
  tests run against those builds in a child process (gcc's ASan runtime
  preloaded, since the Python interpreter is not instrumented).  The 2^32
  exhaustive sweeps and the 2^28-pair algebra run take minutes uninstrumented;
  their sampled versions run instead.
* The C-ABI layer (the library's argument validation, api.hip) is rebuilt with
  clang's sanitizers on its host side only, linked against stand-ins for the
  kernel launchers (tests/native/abi_stubs.hip: on a machine without a GPU no
  call gets past validation), and the C-ABI tests run against that build.

Any sanitizer report aborts the child process, which fails the test.  No GPU
code is built with a sanitizer.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _child(env_extra, args, timeout=900):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *args], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    return out


def _gcc_shared(src, out):
    subprocess.run(["gcc", "-std=c99", "-O1", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    *GCC_SAN, "-o", out, src, "-lm"], check=True)


def test_oracle_and_pins_under_asan_and_ubsan(tmp_path):
    oracle_so = str(tmp_path / "liboracle_san.so")
    pins_so = str(tmp_path / "libpins_san.so")
    _gcc_shared(os.path.join(ROOT, "oracle", "oracle.c"), oracle_so)
    _gcc_shared(os.path.join(ROOT, "tests", "native", "pins.c"), pins_so)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    out = _child({"LD_PRELOAD": libasan, "ORACLE_LIB_OVERRIDE": oracle_so, "PINS_LIB_OVERRIDE": pins_so},
                 ["tests/test_oracle_split.py", "tests/test_oracle_gemm.py", "-m", "not gpu",
                  "-k", "not exhaustive_all_encodings and not random_pairs and not products_exact_exhaustive"])
    assert " passed" in out


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    runtime = _clang_asan_runtime()
    if runtime is None or not os.path.exists(HIPCC):
        pytest.skip("no clang sanitizer runtime or hipcc")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-fno-gpu-flush-denormals-to-zero", "-mcode-object-version=5",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in (os.path.join(ROOT, "fp32_emulated_gemm_amd", "csrc", "api.hip"),
                os.path.join(ROOT, "tests", "native", "abi_stubs.hip")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", "-o", obj, src], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    lib = str(tmp_path / "libsgemm_emu_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-o", lib, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    out = _child({"LD_PRELOAD": runtime, "SGEMM_EMU_LIB_OVERRIDE": lib}, ["tests/test_abi.py", "-m", "not gpu"])
    assert " passed" in out
