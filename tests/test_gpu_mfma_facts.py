"""Hardware facts the GEMM relies on, measured through the library itself.

With BF16-exact inputs and one band (nbands = 1) the product is the plain
sum of x0 y0 over K, as the matrix unit computes it: one
v_mfma_f32_32x32x16_bf16 per 16 consecutive k, each added to the running
result.  The cases below pin what gfx950 does there (observed, then fixed
here so that a change of hardware, compiler flags or denormal mode shows up):

* within one 16-term MFMA sum the products are aligned to the largest one,
  bits more than 24 places below its leading bit are dropped, and the
  aligned sum is rounded once to nearest-even;
* the running result (the MFMA's C operand) is added to that sum exactly and
  rounded once to nearest-even;
* FP32-subnormal products are kept (gradual underflow, ties to even), BF16
  subnormal inputs are not flushed;
* Inf x 0 gives NaN, an overflowing product +Inf.

None of this leaves the elementwise bound the parity tests use: the dropped
bits of a 16-term sum are below 15 * 2^-24 of its largest product, while the
bound allows 2 K 2^-24 sum |a b|.
"""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def fe():
    import fp32_emulated_gemm_amd as fe
    return fe


def dot_bits(fe, a, b):
    """C = a . b (1 x K times K x 1) through sgemm_emu with one band; the FP32 bits."""
    K = len(a)
    print(f"mfma fact K={K}", flush=True, file=sys.stderr)
    A = torch.tensor(np.array(a, np.float32).reshape(1, K), device="cuda")
    B = torch.tensor(np.array(b, np.float32).reshape(K, 1), device="cuda")
    C = torch.full((1, 1), float("nan"), device="cuda")
    fe.sgemm_emu(1, 1, K, A, K, B, 1, C, 1, 1)
    return int(C.cpu().numpy().view(np.uint32)[0, 0])


def bits(x):
    return int(np.float32(x).view(np.uint32))


CASES = [
    # (name, a, b, expected FP32 bits, what it shows)
    ("1 + 1.5u in one sum", [1, 1.5 * U], [1, 1], bits(1.0),
     "2^-25 part dropped (24 places below 1), then 1 + 2^-24 ties to even"),
    ("1 + 3 x 0.375u in one sum", [1] + [0.375 * U] * 3, [1] * 4, bits(1.0),
     "all three terms lie below 2^-24: dropped (nearest of the exact sum would be 1 + 2^-23)"),
    ("2^30 + 1 - 2^30", [2.0 ** 30, 1, -(2.0 ** 30)], [1, 1, 1], bits(0.0),
     "the 1 lies 30 places below the largest product: dropped"),
    ("1 + 2^30 - 2^30", [1, 2.0 ** 30, -(2.0 ** 30)], [1, 1, 1], bits(0.0), "the same in another order"),
    ("2^24 + 15 x 1", [2.0 ** 24] + [1.0] * 15, [1] * 16, bits(2.0 ** 24 + 16),
     "exact 2^24 + 15 is a tie: rounded to even (truncation would give 2^24 + 14)"),
    ("1, then 1.5u in the next sum", [1] + [0] * 15 + [1.5 * U], [1] * 17, bits(1.0 + 2 * U),
     "running result + next sum: exact, then nearest (1 + 2^-23)"),
    ("1, then 0.5u + 0.5u in the next sum", [1] + [0] * 15 + [0.5 * U, 0.5 * U], [1] * 18, bits(1.0),
     "next sum is exactly 2^-24: 1 + 2^-24 ties to even"),
    ("1, then 1.5u two K steps later", [1] + [0] * 31 + [1.5 * U], [1] * 33, bits(1.0 + 2 * U),
     "the same across a K step of the kernel"),
    ("product 2^-140", [2.0 ** -70], [2.0 ** -70], bits(2.0 ** -140), "subnormal product kept"),
    ("product 2^-149", [2.0 ** -75], [2.0 ** -74], 1, "smallest subnormal kept"),
    ("product 2^-150", [2.0 ** -75], [2.0 ** -75], 0, "half the smallest subnormal: tie to even (zero)"),
    ("product 1.5 x 2^-149", [1.5 * 2.0 ** -75], [2.0 ** -74], 2, "tie to even upward"),
    ("BF16 subnormal 2^-130 x 2^100", [2.0 ** -130], [2.0 ** 100], bits(2.0 ** -30), "subnormal input kept"),
    ("BF16 subnormal 2^-133 x 2^120", [2.0 ** -133], [2.0 ** 120], bits(2.0 ** -13), "smallest BF16 subnormal kept"),
    ("2^100 x 2^100", [2.0 ** 100], [2.0 ** 100], bits(np.inf), "overflow gives +Inf"),
]


@pytest.mark.parametrize("name,a,b,expected,why", CASES, ids=[c[0] for c in CASES])
def test_mfma_fact(fe, name, a, b, expected, why):
    got = dot_bits(fe, a, b)
    assert got == expected, f"{name}: got {got:#010x}, expected {expected:#010x} ({why})"


def test_inf_times_zero_is_nan(fe):
    got = np.uint32(dot_bits(fe, [np.inf], [0.0])).view(np.float32)
    assert np.isnan(got)
