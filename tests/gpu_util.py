"""Helpers for the GPU parity tests: device transfers, the error-bound checks and
the exact-class certificate.  The expected values always come from the oracle.

Bounds (acceptance criteria of this build, derived from the pages' claim that
BF16x9 matched or beat native FP32 accuracy against an FP64 reference --
NVIDIA blog, "Limitations and decision criteria"):
  elementwise  |C - C_ref| <= 2 K 2^-24 G + 9 K 2^-149,  G = sum_k |a b|;
  normwise     ||C - C_ref||_F / ||C_ref||_F <= 2 x the same for naive FP32.
"""
import numpy as np
import torch

import oracle

U = 2.0 ** -24
FLOOR = 2.0 ** -149


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def elementwise_bound(K, G):
    return 2.0 * K * U * G + 9.0 * K * FLOOR


def check_against_fp64(C, A, B, rows=None, label="", normwise=True):
    """Assert the elementwise bound on every finite reference element and the
    normwise gate; returns (max ratio to bound, normwise error, naive error)."""
    K = A.shape[1]
    ref, G = oracle.gemm_f64(A, B, rows=rows)
    Cd = C.astype(np.float64)
    err = np.abs(Cd - ref)
    bound = elementwise_bound(K, G)
    finite = np.isfinite(ref)
    bad = finite & ~(err <= bound)
    assert not bad.any(), (f"{label}: {int(bad.sum())} elements exceed the bound; worst "
                           f"{np.nanmax(np.where(finite, err / np.maximum(bound, 1e-300), 0)):.3g}x")
    ratio = float(np.max(np.where(finite, err / np.maximum(bound, 1e-300), 0.0))) if err.size else 0.0
    e_emu = e_naive = 0.0
    if normwise and ref.size:
        naive = oracle.sgemm_naive_f32(A, B, rows=rows).astype(np.float64)
        nref = np.linalg.norm(ref)
        if nref == 0:
            assert np.all(Cd == 0), f"{label}: reference is zero but C is not"
        else:
            e_emu = float(np.linalg.norm(Cd - ref) / nref)
            e_naive = float(np.linalg.norm(naive - ref) / nref)
            assert e_emu <= 2.0 * e_naive, f"{label}: normwise {e_emu:.3g} > 2 x naive {e_naive:.3g}"
    return ratio, e_emu, e_naive


def check_full(label, A, B, C, ablations=None, chunk_elems=1 << 25, keep_ref=None):
    """check_against_fp64 on every element of C = A B, computed in row chunks so the
    FP64 reference, G and the naive FP32 comparator never need to be held whole.

    Asserts the elementwise bound on every finite reference element of every chunk
    and the normwise gate over the whole matrix.  `ablations` maps nbands -> a
    band-drop result of the same product, each held to |C_b - C_ref| <=
    (dropped-mass bound_b + 2 K 2^-24) G + 9 K 2^-149.  `keep_ref(r0, r1, ref)`,
    if given, receives each chunk's FP64 reference (rows r0..r1-1).
    Returns (max ratio to the bound, normwise error, naive normwise error)."""
    M, K = A.shape
    N = B.shape[1]
    rows_per = max(1, min(M, chunk_elems // max(N, 1)))
    drop = {4: 2.0 ** -30, 3: 2.0 ** -21 + 2.0 ** -30, 2: 2.0 ** -13 + 2.0 ** -21 + 2.0 ** -30}
    sq_emu = sq_naive = sq_ref = 0.0
    worst = 0.0
    for r0 in range(0, M, rows_per):
        r1 = min(M, r0 + rows_per)
        rows = np.arange(r0, r1, dtype=np.int64)
        ref, G = oracle.gemm_f64(A, B, rows=rows)
        if keep_ref is not None:
            keep_ref(r0, r1, ref)
        Cd = C[r0:r1].astype(np.float64)
        err = np.abs(Cd - ref)
        bound = elementwise_bound(K, G)
        finite = np.isfinite(ref)
        bad = finite & ~(err <= bound)
        assert not bad.any(), (f"{label}: {int(bad.sum())} elements of rows {r0}..{r1 - 1} exceed the bound; "
                               f"first at {np.argwhere(bad)[0] + [r0, 0]}")
        worst = max(worst, float(np.max(np.where(finite, err / np.maximum(bound, 1e-300), 0.0))))
        for nb, Cb in (ablations or {}).items():
            eb = np.abs(Cb[r0:r1].astype(np.float64) - ref)
            bb = (drop[nb] + 2.0 * K * U) * G + 9.0 * K * FLOOR
            badb = finite & ~(eb <= bb)
            assert not badb.any(), f"{label} nbands={nb}: {int(badb.sum())} elements of rows {r0}..{r1 - 1} exceed"
        naive = oracle.sgemm_naive_f32(A, B, rows=rows).astype(np.float64)
        fin = np.where(finite, 1.0, 0.0)
        sq_emu += float(np.sum(np.where(finite, (Cd - ref) ** 2, 0.0)))
        sq_naive += float(np.sum(np.where(finite, (naive - ref) ** 2, 0.0)))
        sq_ref += float(np.sum(np.where(finite, ref, 0.0) ** 2))
        del ref, G, Cd, err, bound, naive, fin
    if sq_ref == 0.0:
        assert np.all(C == 0), f"{label}: reference is zero but C is not"
        return worst, 0.0, 0.0
    e_emu, e_naive = (sq_emu / sq_ref) ** 0.5, (sq_naive / sq_ref) ** 0.5
    assert e_emu <= 2.0 * e_naive, f"{label}: normwise {e_emu:.3g} > 2 x naive {e_naive:.3g}"
    return worst, e_emu, e_naive


def _lsb_exponents(v):
    """Exponent of the lowest set bit of each nonzero double (0 -> huge)."""
    m, e = np.frexp(v)
    ints = np.abs(np.ldexp(m, 53)).astype(np.int64)
    ints = np.where(ints == 0, 1, ints)
    tz = np.zeros(v.shape, dtype=np.int64)
    x = ints.copy()
    for _ in range(64):
        even = (x & 1) == 0
        if not even.any():
            break
        tz += even
        x = np.where(even, x >> 1, x)
    out = e.astype(np.int64) - 53 + tz
    return np.where(v == 0, 1 << 30, out)


def exact_class_mask(A, B):
    """Elements whose five band sums are exact in any summation order.

    For each band s and element (i, j) the terms A_p[i,k] B_q[k,j] (p + q = s,
    components from the oracle's split) are exact doubles; if all are multiples
    of one quantum 2^e and their absolute sum is below 2^(24+e), every partial
    sum in FP32 is exact.  Elements certified for all five bands must then
    agree bit for bit between any two correct implementations, because the
    recombination is the same sequence of correctly rounded FP32 operations.
    """
    Ac = [np.array(c, np.uint32).__lshift__(16).view(np.float32).astype(np.float64) for c in oracle.split(A)]
    Bc = [np.array(c, np.uint32).__lshift__(16).view(np.float32).astype(np.float64) for c in oracle.split(B)]
    M, K = A.shape
    N = B.shape[1]
    ok = np.ones((M, N), dtype=bool)
    for s in range(5):
        lsb = np.full((M, N), 1 << 30, dtype=np.int64)
        mag = np.zeros((M, N))
        for p in range(3):
            q = s - p
            if not 0 <= q < 3:
                continue
            T = Ac[p][:, :, None] * Bc[q][None, :, :]          # M x K x N, exact
            lsb = np.minimum(lsb, _lsb_exponents(T).min(axis=1))
            mag += np.abs(T).sum(axis=1)
        nonzero = lsb < (1 << 29)
        cert = ~nonzero | (mag * (1 + 2.0 ** -40) < np.ldexp(1.0, np.minimum(lsb, 900) + 24))
        ok &= cert
    return ok
