"""Seeded synthetic inputs for the emulated-SGEMM workloads.

This module only draws random numbers and arranges them into matrices.  It
holds none of the GEMM method's arithmetic (no split, no products, no bands)
and imports neither the GPU library nor the oracle; both sides receive the
arrays it returns.

Random source: numpy's Philox-4x64 counter-based generator.  A matrix is drawn
in fixed blocks of rows; block c uses ``Philox(key=seed).jumped(c)``, so the
values do not depend on how many threads draw them.

Workloads (sizes from the PET-like and square configurations; the PET shapes
stand in for the linear layers of the 192-atom and 17,280-atom water systems
of NVIDIA's blog post "Unlocking Tensor Core Performance for Machine Learning
Interatomic Potentials", section "Benchmarking on PET"):

  square256   A, B 256x256 i.i.d. N(0,1)
  pet_small   X 6144x256 N(0,1); W1 256x1024 N(0,1/256); W2 1024x256 N(0,1/1024)
              (hidden layer H = GELU(X W1) is built by the caller)
  square4096  A, B 4096x4096 i.i.d. U(-1,1)
  pet_large   X 552960x256 N(0,1); W1, W2 as pet_small (hidden layer
              H = GELU(X W1) is built by the caller, as for pet_small)
  stress8192  A, B 8192x8192, entries z 2^u (z ~ N(0,1), u uniform integer in
              [-20, 20]); 1% of A's rows rebuilt as near-cancelling partners of
              other rows, row_j = fp32(-row_i + 2^-20 n); 0.1% of the entries of A
              and of B replaced by random FP32 subnormals
"""
from concurrent.futures import ThreadPoolExecutor
import math
import os

import numpy as np

SEED_BASE = 0x5EED0000
BLOCK_ROWS = 4096

# matrix ids inside a workload (seed = SEED_BASE + 16 * workload_index + matrix_id)
MID_A, MID_B, MID_W2, MID_NOISE, MID_MASK = 0, 1, 2, 3, 4

WORKLOADS = {
    # name: (index, description)
    "square256": 1,
    "pet_small": 2,
    "square4096": 3,
    "pet_large": 4,
    "stress8192": 5,
}

PET_D, PET_FFN, PET_TOKENS = 256, 1024, 32
PET_SMALL_ATOMS, PET_LARGE_ATOMS = 192, 17280


def seed_of(workload: str, matrix_id: int) -> int:
    return SEED_BASE + 16 * WORKLOADS[workload] + matrix_id


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _blocks(rows: int):
    return [(c, c * BLOCK_ROWS, min(rows, (c + 1) * BLOCK_ROWS))
            for c in range((rows + BLOCK_ROWS - 1) // BLOCK_ROWS)]


def _fill(shape, seed, draw):
    """Fill a float32 matrix block by block; draw(gen, nrows, ncols) -> float32 block."""
    rows, cols = shape
    out = np.empty((rows, cols), dtype=np.float32)
    base = np.random.Philox(key=seed)

    def work(blk):
        c, r0, r1 = blk
        gen = np.random.Generator(base.jumped(c))
        out[r0:r1] = draw(gen, r1 - r0, cols)

    blocks = _blocks(rows)
    if len(blocks) > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, blocks))
    elif blocks:
        work(blocks[0])
    return out


def normal(shape, sigma: float, seed: int) -> np.ndarray:
    """fp32_RNE(sigma * z), z ~ N(0,1) drawn in double."""
    return _fill(shape, seed, lambda g, r, c: (sigma * g.standard_normal((r, c))).astype(np.float32))


def uniform(shape, seed: int) -> np.ndarray:
    """fp32_RNE(2u - 1), u ~ U[0,1) with 53 random bits."""
    return _fill(shape, seed, lambda g, r, c: (2.0 * g.random((r, c)) - 1.0).astype(np.float32))


def scaled_normal(shape, seed: int, umin: int = -20, umax: int = 20) -> np.ndarray:
    """Entries z * 2^u with z ~ N(0,1) and u a uniform integer in [umin, umax]."""
    def draw(g, r, c):
        z = g.standard_normal((r, c))
        u = g.integers(umin, umax + 1, size=(r, c))
        return np.ldexp(z, u).astype(np.float32)
    return _fill(shape, seed, draw)


def subnormal_sprinkle(X: np.ndarray, fraction: float, seed: int) -> np.ndarray:
    """Replace a random `fraction` of X's entries by random FP32 subnormals in place.

    Each replaced entry has a random sign and a mantissa uniform in [1, 2^23 - 1]
    with a zero exponent field.
    """
    g = np.random.Generator(np.random.Philox(key=seed))
    n = int(round(fraction * X.size))
    if n == 0:
        return X
    idx = g.choice(X.size, size=n, replace=False)
    mant = g.integers(1, 1 << 23, size=n, dtype=np.uint32)
    sign = g.integers(0, 2, size=n, dtype=np.uint32) << np.uint32(31)
    X.reshape(-1).view(np.uint32)[idx] = sign | mant
    return X


def near_cancelling_rows(X: np.ndarray, fraction: float, seed: int, noise_seed: int):
    """Rebuild a `fraction` of X's rows as row_j = fp32(-row_i + 2^-20 n), n ~ N(0,1).

    Each target row j is paired with a distinct source row i that is left
    untouched.  Returns the (source, target) index arrays.
    """
    M, K = X.shape
    npairs = int(round(fraction * M))
    if npairs == 0 or 2 * npairs > M:
        return np.empty(0, np.int64), np.empty(0, np.int64)
    g = np.random.Generator(np.random.Philox(key=seed))
    picked = g.choice(M, size=2 * npairs, replace=False)
    src, dst = picked[:npairs], picked[npairs:]
    noise = np.random.Generator(np.random.Philox(key=noise_seed)).standard_normal((npairs, K))
    X[dst] = (-X[src].astype(np.float64) + np.ldexp(noise, -20)).astype(np.float32)
    return src.astype(np.int64), dst.astype(np.int64)


# --------------------------------------------------------------------------- workloads

def square256(n: int = 256):
    w = "square256"
    return {"A": normal((n, n), 1.0, seed_of(w, MID_A)),
            "B": normal((n, n), 1.0, seed_of(w, MID_B))}


def pet_weights(workload: str, d: int = PET_D, ffn: int = PET_FFN):
    """W1 [d x ffn] ~ N(0, 1/d) and W2 [ffn x d] ~ N(0, 1/ffn)."""
    return {"W1": normal((d, ffn), 1.0 / math.sqrt(d), seed_of(workload, MID_B)),
            "W2": normal((ffn, d), 1.0 / math.sqrt(ffn), seed_of(workload, MID_W2))}


def pet_small(atoms: int = PET_SMALL_ATOMS):
    w = "pet_small"
    out = {"X": normal((atoms * PET_TOKENS, PET_D), 1.0, seed_of(w, MID_A))}
    out.update(pet_weights(w))
    return out


def pet_large(atoms: int = PET_LARGE_ATOMS):
    w = "pet_large"
    rows = atoms * PET_TOKENS
    out = {"X": normal((rows, PET_D), 1.0, seed_of(w, MID_A))}
    out.update(pet_weights(w))
    return out


def square4096(n: int = 4096):
    w = "square4096"
    return {"A": uniform((n, n), seed_of(w, MID_A)),
            "B": uniform((n, n), seed_of(w, MID_B))}


def stress8192(n: int = 8192, k: int = None, m: int = None):
    """Accuracy stress: scaled normals, near-cancelling row pairs, subnormal sprinkle."""
    w = "stress8192"
    m = n if m is None else m
    k = n if k is None else k
    A = scaled_normal((m, k), seed_of(w, MID_A))
    B = scaled_normal((k, n), seed_of(w, MID_B))
    src, dst = near_cancelling_rows(A, 0.01, seed_of(w, MID_MASK), seed_of(w, MID_NOISE))
    subnormal_sprinkle(A, 0.001, seed_of(w, MID_MASK) + 1000)
    subnormal_sprinkle(B, 0.001, seed_of(w, MID_MASK) + 2000)
    return {"A": A, "B": B, "pair_src": src, "pair_dst": dst}
