"""Pins of the oracle's split and of the BF16-product premise (CPU only).

Split rule: NVIDIA Technical Blog "Unlocking Tensor Core Performance for Machine
Learning Interatomic Potentials", Fig. 1 caption; discuss.pytorch.kr summary,
BF16x9 section (x = x0 + 2^-8 x1 + 2^-16 x2, 8 significant bits per piece).
"""
import ctypes
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden(name="split_cases.txt"):
    rows = []
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            parts = line.split()
            rows.append(tuple(int(p, 16) for p in parts[:4]))
    return rows


@pytest.mark.parametrize("case", _golden(), ids=lambda c: f"{c[0]:08X}")
def test_split_golden(orc, case):
    u, e0, e1, e2 = case
    x = np.array([u], dtype=np.uint32).view(np.float32)
    c = orc.split(x)
    assert (int(c[0][0]), int(c[1][0]), int(c[2][0])) == (e0, e1, e2)
    assert orc.split_one(float(x[0])) == (e0, e1, e2) or np.isnan(x[0])


@pytest.mark.parametrize("case", _golden("split_rne_cases.txt"), ids=lambda c: f"{c[0]:08X}")
def test_split_rne_golden(orc, case):
    """The round-to-nearest-even split (rounding ablation) on hand-derived cases."""
    u, e0, e1, e2 = case
    x = np.array([u], dtype=np.uint32).view(np.float32)
    c = orc.split(x, orc.SPLIT_RNE)
    assert (int(c[0][0]), int(c[1][0]), int(c[2][0])) == (e0, e1, e2)


def test_split_rne_exhaustive_all_encodings(orc, pins):
    """Every FP32 encoding through the round-to-nearest split: exact
    reconstruction, nearest-even BF16 at both stages (never Inf), special classes."""
    chunk = 1 << 26
    first = ctypes.c_uint64()
    for start in range(0, 1 << 32, chunk):
        x = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        c0, c1, c2 = orc.split(x, orc.SPLIT_RNE)
        bad = pins.pin_split_rne_range(start, chunk, c0.ctypes.data, c1.ctypes.data, c2.ctypes.data,
                                       ctypes.byref(first))
        assert bad == 0, f"{bad} encodings fail from {start:#x}; first {first.value:#010x}"


@pytest.mark.parametrize("rne", [False, True])
def test_split_sampled_encodings(orc, pins, rne):
    """The checks of the exhaustive tests on 256 runs of 2^14 consecutive
    encodings spread over the whole space (every exponent, both signs, the
    special classes): a fast version, also run under the sanitizers."""
    first = ctypes.c_uint64()
    run = 1 << 14
    for i in range(256):
        start = (i << 24) + (i * 40503 % (1 << 24 - 14)) * run
        x = np.arange(start, start + run, dtype=np.uint64).astype(np.uint32).view(np.float32)
        c0, c1, c2 = orc.split(x, orc.SPLIT_RNE if rne else orc.SPLIT_RZ)
        check = pins.pin_split_rne_range if rne else pins.pin_split_range
        bad = check(start, run, c0.ctypes.data, c1.ctypes.data, c2.ctypes.data, ctypes.byref(first))
        assert bad == 0, f"{bad} encodings fail from {start:#x}; first {first.value:#010x}"


def test_split_shapes_and_strides(orc):
    X = np.arange(12, dtype=np.float32).reshape(3, 4) * np.float32(1.0009765625)
    c = orc.split(X)
    assert all(ci.shape == (3, 4) and ci.dtype == np.uint16 for ci in c)
    e = orc.split(np.zeros((0, 5), np.float32))
    assert e[0].shape == (0, 5)


def test_split_exhaustive_all_encodings(orc, pins):
    """Every one of the 2^32 FP32 encodings: exact reconstruction, RZ per stage,
    signs, special classes (checked by tests/native/pins.c)."""
    chunk = 1 << 26
    total_bad = 0
    first = ctypes.c_uint64()
    for start in range(0, 1 << 32, chunk):
        x = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        c0, c1, c2 = orc.split(x)
        bad = pins.pin_split_range(start, chunk, c0.ctypes.data, c1.ctypes.data, c2.ctypes.data,
                                   ctypes.byref(first))
        assert bad == 0, f"{bad} encodings fail from {start:#x}; first {first.value:#010x}"
        total_bad += bad
    assert total_bad == 0


def test_bf16_products_exact_exhaustive(pins):
    """All 2^32 ordered BF16 pairs: the FP32 product equals the exact product
    whenever it lies in FP32's normal range (the premise of evaluating the
    pairwise products on BF16 matrix units with FP32 accumulation)."""
    checked = ctypes.c_int64()
    total = 0
    for a0 in range(0, 65536, 8192):
        bad = pins.pin_bf16_products(a0, 8192, ctypes.byref(checked))
        assert bad == 0
        total += checked.value
    assert total > 3_000_000_000


def _random_floats(g, n):
    """Random finite FP32 values over the whole exponent range, incl. subnormals."""
    u = g.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    expo = (u >> np.uint32(23)) & np.uint32(0xFF)
    u = np.where(expo == 0xFF, u & np.uint32(0x807FFFFF) | np.uint32(0x3F800000), u)
    return u.view(np.float32)


def test_band_algebra_random_pairs(orc, pins):
    """Exact nine-term identity, the omitted-term identity of the TF32x3 form, and
    the dropped-mass bounds per band count, on 2^28 random pairs drawn over the
    whole FP32 range (products kept inside double's exact range)."""
    g = np.random.Generator(np.random.Philox(key=0xA16EB7A))
    n = 1 << 24
    for _ in range(16):
        a = _random_floats(g, n)
        b = _random_floats(g, n)
        # keep |a*b| away from FP32 overflow/underflow only where needed: double holds all
        ca, cb = orc.split(a), orc.split(b)
        bad = pins.pin_band_algebra(n, a.ctypes.data, b.ctypes.data,
                                    *[c.ctypes.data for c in ca], *[c.ctypes.data for c in cb])
        assert bad == 0


def test_band_algebra_special_classes(orc, pins):
    """Zeros, subnormals, FLT_MIN/FLT_MAX neighbours and powers of two."""
    vals = [0.0, -0.0, 1.0, -1.0, 2.0 ** -126, 2.0 ** -149, -(2.0 ** -149), 3.4028234663852886e38,
            1.1754942106924411e-38, 1.0000001192092896, 0.99999994039535522, 2.0 ** 100, 2.0 ** -100,
            3.1415927410125732, -2.7182817459106445]
    v = np.array(vals, dtype=np.float32)
    a = np.repeat(v, v.size)
    b = np.tile(v, v.size)
    ca, cb = orc.split(a), orc.split(b)
    bad = pins.pin_band_algebra(a.size, a.ctypes.data, b.ctypes.data,
                                *[c.ctypes.data for c in ca], *[c.ctypes.data for c in cb])
    assert bad == 0
