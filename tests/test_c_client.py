"""The C ABI from a plain C program, on the CPU: include/sgemm_emu.h compiles as
strict C99 and as C++17 with every warning an error, a C client links against
the built library and its calls that need no GPU (the product count, argument
validation of the split-K queries, the status strings) return what the header
states."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "fp32_emulated_gemm_amd")

CLIENT = r"""
#include <stdio.h>
#include "sgemm_emu.h"
int main(void)
{
    int b;
    for (b = 1; b <= 5; ++b) printf("%d ", sgemm_emu_products(b));
    printf("| %d %d %d %d | %s | %s\n", sgemm_emu_split_k(4, 4, 4, 0), sgemm_emu_split_k(-1, 4, 4, 5),
           sgemm_emu_split_k_fp32_b(4, 4, 4, 6), sgemm_emu_split_k_fp32_b(4, -4, 4, 5),
           sgemm_emu_strerror(SGEMM_EMU_EINVAL), sgemm_emu_strerror(SGEMM_EMU_OK));
    return 0;
}
"""


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("no host C compiler")
    d = tmp_path_factory.mktemp("cclient")
    src = d / "client.c"
    src.write_text(CLIENT)
    inc = os.path.join(ROOT, "include")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", inc, "-c", str(src), "-o",
                    str(d / "client.o")], check=True)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-I", inc, "-x", "c++", "-c", str(src),
                    "-o", str(d / "client_cxx.o")], check=True)
    exe = d / "client"
    subprocess.run(["gcc", str(d / "client.o"), "-L", LIBDIR, "-lsgemm_emu", "-Wl,-rpath," + LIBDIR, "-o", str(exe)],
                   check=True)
    return exe


def test_header_compiles_and_c_client_runs(client):
    env = dict(os.environ)
    if os.path.isdir("/opt/rocm/lib"):
        env["LD_LIBRARY_PATH"] = "/opt/rocm/lib" + (":" + env["LD_LIBRARY_PATH"] if env.get("LD_LIBRARY_PATH") else "")
    r = subprocess.run([str(client)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stderr
    products, queries, einval, ok = [x.strip() for x in r.stdout.split("|")]
    assert products.split() == ["1", "3", "6", "8", "9"]
    assert queries.split() == ["-1", "-1", "-1", "-1"]          # SGEMM_EMU_EINVAL before any HIP call
    assert "invalid argument" in einval
    assert ok
