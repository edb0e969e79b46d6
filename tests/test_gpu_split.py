"""GPU split kernel vs the oracle's split: bit-exact (through the C ABI)."""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fe():
    import fp32_emulated_gemm_amd as fe
    return fe


def _planes_host(planes):
    torch.cuda.synchronize()
    return [p.cpu().numpy().view(np.uint16) for p in planes]


def test_split_all_encodings_bit_exact(fe, orc):
    """All 2^32 FP32 encodings, in chunks of 2^28, through split_f32_bf16x3."""
    chunk = 1 << 28
    for start in range(0, 1 << 32, chunk):
        print(f"split chunk {start:#x}", flush=True, file=sys.stderr)
        x = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda").to(torch.int32).view(torch.float32)
        planes = [torch.empty(chunk, dtype=torch.int16, device="cuda") for _ in range(3)]
        fe.split_f32_bf16x3(1, chunk, x, chunk, *planes, chunk)
        got = _planes_host(planes)
        xh = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        want = orc.split(xh)
        for c in range(3):
            if not np.array_equal(got[c], want[c]):
                bad = np.nonzero(got[c] != want[c])[0][0]
                raise AssertionError(f"component {c} differs at encoding {start + bad:#010x}: "
                                     f"gpu {got[c][bad]:#06x} oracle {want[c][bad]:#06x}")
        del x, planes


@pytest.mark.parametrize("rows,cols,ldx,ldo,offset", [
    (37, 53, 53, 53, 0),        # odd widths: scalar kernel
    (64, 256, 256, 256, 0),     # contiguous: folded vector kernel
    (33, 64, 72, 80, 0),        # strided rows, vector kernel
    (16, 40, 41, 40, 1),        # misaligned start: scalar kernel
    (1, 8, 8, 8, 0),
])
def test_split_layouts(fe, orc, rows, cols, ldx, ldo, offset):
    g = np.random.Generator(np.random.Philox(key=rows * 1000 + cols))
    buf = (g.standard_normal(rows * ldx + offset + 8) * 2.0 ** g.integers(-60, 60, rows * ldx + offset + 8))
    buf = buf.astype(np.float32)
    X = torch.from_numpy(buf).cuda()
    Xv = X[offset:offset + rows * ldx].view(rows, ldx)
    planes = [torch.full((rows * ldo,), -1, dtype=torch.int16, device="cuda") for _ in range(3)]
    fe.split_f32_bf16x3(rows, cols, Xv, ldx, *planes, ldo)
    got = [p.reshape(rows, ldo) for p in _planes_host(planes)]
    want = orc.split(buf[offset:offset + rows * ldx].reshape(rows, ldx)[:, :cols])
    for c in range(3):
        assert np.array_equal(got[c][:, :cols], want[c])
        if ldo > cols:
            assert np.all(got[c][:, cols:] == 0xFFFF)   # padding untouched


def test_split_empty_is_noop(fe):
    fe.split_f32_bf16x3(0, 16, None, 16, None, None, None, 16)


@pytest.mark.parametrize("rows,cols,ldx,ldo", [
    (64, 64, 64, 64),           # small: 32 x 32 LDS tiles
    (256, 1024, 1024, 256),     # a [out][in] weight, 32 x 32 tiles
    (1024, 257, 260, 1032),     # ragged columns, padded leading dimensions
    (1024, 1024, 1024, 1024),   # 64 x 64 LDS tiles (at least one per CU)
    (2048, 520, 530, 2056),     # 64 x 64 tiles, ragged, padded
    (130, 70, 70, 130),         # rows not a multiple of 8: scalar kernel
    (24, 5, 7, 40),
])
def test_split_transposed_bit_exact(fe, orc, rows, cols, ldx, ldo):
    """split_f32_bf16x3_transposed(X) == the oracle's split of X^T, including
    Inf, NaN, zeros and subnormals; padding of the planes untouched."""
    g = np.random.Generator(np.random.Philox(key=rows * 7 + cols))
    X = (g.standard_normal((rows, ldx)) * 2.0 ** g.integers(-60, 60, (rows, ldx))).astype(np.float32)
    specials = [np.inf, -np.inf, np.nan, 0.0, -0.0, np.float32(1e-41), np.float32(-3e-39)]
    for s, v in enumerate(specials):
        X[(s * 5) % rows, (s * 3) % cols] = v
    print(f"split transposed {rows}x{cols} ldx={ldx} ldo={ldo}", flush=True, file=sys.stderr)
    planes = [torch.full((cols * ldo,), -1, dtype=torch.int16, device="cuda") for _ in range(3)]
    fe.split_f32_bf16x3_transposed(rows, cols, torch.from_numpy(X).cuda(), ldx, *planes, ldo)
    got = [p.reshape(cols, ldo) for p in _planes_host(planes)]
    want = orc.split(np.ascontiguousarray(X[:, :cols].T))
    for c in range(3):
        assert np.array_equal(got[c][:, :rows], want[c])
        if ldo > rows:
            assert np.all(got[c][:, rows:] == 0xFFFF)


def test_split_rne_all_encodings_bit_exact(fe, orc):
    """The round-to-nearest split (SGEMM_EMU_SPLIT_RNE) on all 2^32 encodings."""
    chunk = 1 << 28
    for start in range(0, 1 << 32, chunk):
        print(f"split rne chunk {start:#x}", flush=True, file=sys.stderr)
        x = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda").to(torch.int32).view(torch.float32)
        planes = [torch.empty(chunk, dtype=torch.int16, device="cuda") for _ in range(3)]
        fe.split_f32_bf16x3_ex(1, chunk, x, chunk, *planes, chunk, fe.SGEMM_EMU_SPLIT_RNE)
        got = _planes_host(planes)
        xh = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        want = orc.split(xh, orc.SPLIT_RNE)
        for c in range(3):
            if not np.array_equal(got[c], want[c]):
                bad = np.nonzero(got[c] != want[c])[0][0]
                raise AssertionError(f"rne component {c} differs at encoding {start + bad:#010x}: "
                                     f"gpu {got[c][bad]:#06x} oracle {want[c][bad]:#06x}")
        del x, planes


@pytest.mark.parametrize("rows,cols,ldx,ldo,flags", [
    (37, 53, 53, 53, 1),        # scalar kernel, RNE
    (64, 256, 256, 256, 1),     # vector kernel, RNE
    (256, 1024, 1024, 256, 3),  # transposed, 32 x 32 tiles, RNE
    (1024, 1024, 1024, 1024, 3),  # transposed, 64 x 64 tiles, RNE
    (130, 70, 70, 130, 3),      # transposed, element-wise, RNE
])
def test_split_ex_layouts(fe, orc, rows, cols, ldx, ldo, flags):
    g = np.random.Generator(np.random.Philox(key=rows * 3 + cols + flags))
    X = (g.standard_normal((rows, ldx)) * 2.0 ** g.integers(-60, 60, (rows, ldx))).astype(np.float32)
    X[1, 2] = np.float32(3.4028235e38)
    tr = bool(flags & fe.SGEMM_EMU_SPLIT_TRANSPOSE)
    prow, pcol = (cols, rows) if tr else (rows, cols)
    planes = [torch.full((prow * ldo,), -1, dtype=torch.int16, device="cuda") for _ in range(3)]
    print(f"split ex {rows}x{cols} flags={flags}", flush=True, file=sys.stderr)
    fe.split_f32_bf16x3_ex(rows, cols, torch.from_numpy(X).cuda(), ldx, *planes, ldo, flags)
    got = [p.reshape(prow, ldo)[:, :pcol] for p in _planes_host(planes)]
    src = X[:, :cols].T if tr else X[:, :cols]
    want = orc.split(np.ascontiguousarray(src), orc.SPLIT_RNE)
    for c in range(3):
        assert np.array_equal(got[c], want[c])
