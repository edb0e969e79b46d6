"""Compile the HIP sources into libsgemm_emu.so (gfx950 only), and the same
sources with -DSGEMM_EMU_SERIAL_LDS into libsgemm_emu_serial_lds.so: a debug
build whose N x K plane GEMM runs a kernel with one LDS buffer per operand and a
barrier on each side of every K step (no stream-K, A split in that kernel); its
results must equal the library's bit for bit where the library runs the
pipelined kernel without stream-K (tests/test_gpu_serial_lds.py).

    python -m fp32_emulated_gemm_amd.build

Flags:
  --offload-arch=gfx950              the only target (MI355X)
  -ffp-contract=off                  no implicit FMA: the split's sub/mul stay exact
                                     and the epilogue's FMAs are written explicitly
  -fno-gpu-flush-denormals-to-zero   FP32 subnormals kept (the split is exact for them)
  -target-feature -packed-fp32-ops   keep the compiler from emitting packed FP32 ops
  -mcode-object-version=5            loadable by the ROCm runtime that PyTorch bundles
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsgemm_emu.so")
DEBUG_LIB = os.path.join(HERE, "libsgemm_emu_serial_lds.so")
SOURCES = ["api.hip", "gemm.hip", "split.hip", "ieee.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero", "-mcode-object-version=5",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Always recompiles both libraries (every source in parallel, then one
    link each); returns the path of the library."""
    with tempfile.TemporaryDirectory(prefix="sgemm_emu_build_") as tmpdir:
        jobs = []
        for lib, extra, tag in ((LIB, [], ""), (DEBUG_LIB, ["-DSGEMM_EMU_SERIAL_LDS"], "_serial")):
            objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + tag + ".o") for s in SOURCES]
            cmds = [[HIPCC, *FLAGS, *extra, "-c", "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
            jobs.append((lib, objs, cmds))
        with ThreadPoolExecutor(max_workers=8) as pool:
            for f in [pool.submit(_run, c, verbose) for _, _, cmds in jobs for c in cmds]:
                f.result()
        for lib, objs, _ in jobs:
            tmp = lib + ".tmp"
            # -Bsymbolic: each library's internal calls bind to its own definitions,
            # also when both are loaded into one process
            _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-Bsymbolic", "-o", tmp, *objs], verbose)
            os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
