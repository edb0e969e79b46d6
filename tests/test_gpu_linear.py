"""Linear layer on the emulated GEMM: forward Y = X W^T + b (sgemm_emu_linear) and
the input gradient dX = dY W (the same weight planes read as K x N), against the
oracle's FP64 products, plus the torch op and module built on them.

Forward bound: the GEMM's elementwise bound plus one FP32 rounding of the bias
add, |Y - (X W^T + b)| <= 2 K 2^-24 G + 9 K 2^-149 + 2^-24 |X W^T + b|.
"""
import sys

import numpy as np
import pytest
import torch

from gpu_util import FLOOR, U, check_against_fp64, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fe():
    import fp32_emulated_gemm_amd as fe
    return fe


def _rng(seed):
    return np.random.Generator(np.random.Philox(key=seed))


def _planes(fe, W):
    return fe.split(dev(W))


def _forward(fe, X, W, b, nbands=5, act=0):
    M, K = X.shape
    N = W.shape[0]
    print(f"linear fwd M={M} N={N} K={K} bias={b is not None} nbands={nbands} act={act}", flush=True,
          file=sys.stderr)
    P = _planes(fe, W)
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    fe.sgemm_emu_linear(M, N, K, dev(X), max(K, 1), *P, max(K, 1), None if b is None else dev(b), act, Y,
                        max(N, 1), nbands)
    return host(Y)


def gelu_tolerance(z, e):
    """Allowed |GELU_gpu - fp32(GELU(z))| at the exact pre-activation z, for an
    FP32 erfc-form evaluation: the rounded argument z/sqrt 2 (2 ulp, amplified
    by |d ln erfc(x)/dx| <= 2|x| + 1.2 in the tail, x = z/sqrt 2), the erfc
    evaluation and the final product (16 ulp in all), the oracle's own rounding,
    plus a floor for results below the normal range."""
    x = np.abs(z) / np.sqrt(2.0)
    return (16.0 + 4.0 * x * (x + 0.6)) * U * np.abs(e) + 2.0 ** -140


LIN_SHAPES = [(1, 1, 1), (37, 70, 33), (300, 257, 128), (1000, 1030, 256), (2048, 1024, 256), (129, 64, 100)]


@pytest.mark.parametrize("shape", LIN_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_with_bias_within_bound(fe, orc, shape):
    M, N, K = shape
    g = _rng(M * 13 + N * 7 + K)
    X = g.standard_normal((M, K)).astype(np.float32)
    W = (g.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    b = g.standard_normal(N).astype(np.float32)
    Y = _forward(fe, X, W, b).astype(np.float64)
    ref, G = orc.gemm_f64(X, np.ascontiguousarray(W.T))
    ref = ref + b.astype(np.float64)[None, :]
    bound = 2.0 * K * U * G + 9.0 * K * FLOOR + U * np.abs(ref)
    assert np.all(np.abs(Y - ref) <= bound)


def test_forward_bias_is_one_rounding_after_the_gemm(fe):
    """Y = fl32(C + b) with C the pre-split N x K GEMM on the same arguments, and
    Y = C bit for bit without a bias."""
    M, N, K = 700, 300, 192
    g = _rng(4)
    X = g.standard_normal((M, K)).astype(np.float32)
    W = g.standard_normal((N, K)).astype(np.float32)
    b = (g.standard_normal(N) * 3).astype(np.float32)
    b[:5] = [0.0, -0.0, np.float32(1e-40), -1e30, 7.0]
    P = _planes(fe, W)
    Cd = torch.empty((M, N), dtype=torch.float32, device="cuda")
    fe.sgemm_emu_presplit_b(M, N, K, dev(X), K, *P, K, fe.SGEMM_EMU_B_NK, Cd, N, 5)
    C = host(Cd)
    assert np.array_equal(_forward(fe, X, W, b).view(np.uint32), (C + b[None, :]).view(np.uint32))
    assert np.array_equal(_forward(fe, X, W, None).view(np.uint32), C.view(np.uint32))


@pytest.mark.parametrize("nbands", [1, 3, 5])
def test_forward_bands_and_k_zero(fe, nbands):
    g = _rng(50 + nbands)
    b = g.standard_normal(40).astype(np.float32)
    b[0] = -0.0
    Y = _forward(fe, np.zeros((9, 0), np.float32), np.zeros((40, 0), np.float32), b, nbands)
    assert np.array_equal(Y.view(np.uint32), np.broadcast_to((np.float32(0) + b), (9, 40)).view(np.uint32))


@pytest.mark.parametrize("shape", [(37, 70, 33), (300, 257, 128), (2048, 1024, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_forward_gelu_epilogue_vs_oracle(fe, orc, shape):
    """Y = GELU(X W^T + b) fused in the epilogue against the oracle's exact GELU of
    its FP64 pre-activation: the GEMM bound carried through GELU (slope <= 1.13)
    plus the evaluation tolerance."""
    M, N, K = shape
    g = _rng(M * 5 + N * 3 + K)
    X = g.standard_normal((M, K)).astype(np.float32)
    W = (g.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    b = (2.0 * g.standard_normal(N)).astype(np.float32)
    Y = _forward(fe, X, W, b, act=fe.SGEMM_EMU_ACT_GELU).astype(np.float64)
    Z, G = orc.gemm_f64(X, np.ascontiguousarray(W.T))
    Z = Z + b.astype(np.float64)[None, :]
    E = orc.gelu_f64_to_f32(Z).astype(np.float64)
    e_gemm = 2.0 * K * U * G + 9.0 * K * FLOOR + U * np.abs(Z)
    assert np.all(np.abs(Y - E) <= 1.13 * e_gemm + gelu_tolerance(Z, E))
    assert (Z < -5).any() and (Z > 5).any()          # both tails exercised


def test_gelu_epilogue_k_zero_and_extremes(fe, orc):
    """K = 0: Y = GELU(0 + b); b spans the far negative tail, zeros and large values."""
    b = np.array([-0.0, 0.0, -12.0, -9.0, -6.0, -3.0, -1.0, -1e-3, 1e-3, 1.0, 3.0, 10.0, 1e30, -1e30, 1e-40],
                 np.float32)
    Y = _forward(fe, np.zeros((3, 0), np.float32), np.zeros((b.size, 0), np.float32), b,
                 act=fe.SGEMM_EMU_ACT_GELU).astype(np.float64)
    z = (np.float32(0) + b).astype(np.float64)
    E = orc.gelu_f64_to_f32(z).astype(np.float64)
    fin = np.isfinite(E)
    assert np.all(np.abs(Y[:, fin] - E[fin]) <= gelu_tolerance(z[fin], E[fin]))
    assert np.all(Y[:, 13] == 0.0) and np.all(Y[:, 12] == np.float32(1e30))


@pytest.mark.parametrize("shape", [(300, 257, 128), (1024, 256, 1024), (77, 1000, 96)],
                         ids=lambda s: "x".join(map(str, s)))
def test_input_gradient_within_bound(fe, shape):
    """dX = dY W through the weight's planes read as K x N (K = out_features)."""
    M, N, K = shape              # layer: in = K, out = N
    g = _rng(M + N + K)
    W = g.standard_normal((N, K)).astype(np.float32)
    dY = g.standard_normal((M, N)).astype(np.float32)
    P = _planes(fe, W)
    dX = torch.empty((M, K), dtype=torch.float32, device="cuda")
    print(f"linear bwd M={M} N={N} K={K}", flush=True, file=sys.stderr)
    fe.sgemm_emu_presplit_b(M, K, N, dev(dY), N, *P, K, fe.SGEMM_EMU_B_KN, dX, K, 5)
    check_against_fp64(host(dX), dY, W, label=f"dX {shape}")


@pytest.mark.parametrize("shape", [(1100, 256, 1024), (300, 130, 64), (77, 1000, 96)],
                         ids=lambda s: "x".join(map(str, s)))
def test_input_gradient_transposed_planes_bitwise(fe, shape):
    """dX = dY W from the planes of W^T (N x K, split_f32_bf16x3_transposed of W)
    equals the K x N reading of W's own planes bit for bit."""
    M, N, K = shape              # layer: in = K, out = N
    g = _rng(3 * M + N + K)
    W = g.standard_normal((N, K)).astype(np.float32)
    dY = g.standard_normal((M, N)).astype(np.float32)
    Wd, dYd = dev(W), dev(dY)
    P = fe.split(Wd)
    T = fe.split_t(Wd)
    a = torch.empty((M, K), dtype=torch.float32, device="cuda")
    b = torch.empty((M, K), dtype=torch.float32, device="cuda")
    print(f"linear bwd planes M={M} N={N} K={K}", flush=True, file=sys.stderr)
    fe.sgemm_emu_presplit_b(M, K, N, dYd, N, *P, K, fe.SGEMM_EMU_B_KN, a, K, 5)
    fe.sgemm_emu_presplit_b(M, K, N, dYd, N, *T, N, fe.SGEMM_EMU_B_NK, b, K, 5)
    check_against_fp64(host(b), dY, W, label=f"dX planes of W^T {shape}")
    # K x N planes go to the N x K kernel through a workspace padded to a multiple
    # of 64; that kernel cuts K (stream-K) on small grids, and so do the caller's
    # N x K planes when N % 64 == 0: compare where both make the same cuts
    npad = (N + 63) // 64 * 64
    if N % 64 == 0 or fe.sgemm_emu_split_k(M, K, npad) == 1:
        assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32))


def test_forward_split_k_with_bias_and_gelu(fe, orc):
    """A small grid (stream-K): bias and GELU are applied by the workgroup that
    adds a tile's K pieces."""
    M, N, K = 200, 140, 1024
    assert fe.sgemm_emu_split_k(M, N, K) > 1
    g = _rng(808)
    X = g.standard_normal((M, K)).astype(np.float32)
    W = (g.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    b = (2.0 * g.standard_normal(N)).astype(np.float32)
    Z, G = orc.gemm_f64(X, np.ascontiguousarray(W.T))
    Z = Z + b.astype(np.float64)[None, :]
    e_gemm = 2.0 * K * U * G + 9.0 * K * FLOOR + U * np.abs(Z)
    Y = _forward(fe, X, W, b).astype(np.float64)
    assert np.all(np.abs(Y - Z) <= e_gemm)
    Yg = _forward(fe, X, W, b, act=fe.SGEMM_EMU_ACT_GELU).astype(np.float64)
    E = orc.gelu_f64_to_f32(Z).astype(np.float64)
    assert np.all(np.abs(Yg - E) <= 1.13 * e_gemm + gelu_tolerance(Z, E))


def test_torch_op_forward_and_input_gradient(fe, orc):
    from fp32_emulated_gemm_amd.linear import linear
    g = _rng(77)
    B, T, K, N = 6, 50, 96, 130
    X = g.standard_normal((B, T, K)).astype(np.float32)
    W = (g.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    b = g.standard_normal(N).astype(np.float32)
    Gy = g.standard_normal((B, T, N)).astype(np.float32)
    x = dev(X).requires_grad_(True)
    y = linear(x, dev(W), dev(b))
    assert y.shape == (B, T, N)
    (y * dev(Gy)).sum().backward()
    Y = host(y.detach()).reshape(-1, N).astype(np.float64)
    ref, G = orc.gemm_f64(X.reshape(-1, K), np.ascontiguousarray(W.T))
    ref += b[None, :]
    assert np.all(np.abs(Y - ref) <= 2.0 * K * U * G + 9.0 * K * FLOOR + U * np.abs(ref))
    check_against_fp64(host(x.grad).reshape(-1, K), Gy.reshape(-1, N), W, label="torch op dX")


def test_torch_op_gelu_forward_only(fe):
    from fp32_emulated_gemm_amd.linear import Linear, linear
    torch.manual_seed(1)
    ref_layer = torch.nn.Linear(96, 40).cuda()
    m = Linear.from_linear(ref_layer)
    m.activation = "gelu"
    x = torch.randn(300, 96, device="cuda")
    with torch.no_grad():
        y = m(x)
        y_ref = torch.nn.functional.gelu(ref_layer(x))
    assert torch.allclose(y, y_ref, rtol=1e-5, atol=1e-6)
    with pytest.raises(NotImplementedError):
        linear(x.requires_grad_(True), m.weight, m.bias, activation="gelu")
    with pytest.raises(ValueError):
        linear(x.detach(), m.weight, m.bias, activation="relu")


def test_module_matches_nn_linear_and_refuses_parameter_grads(fe):
    from fp32_emulated_gemm_amd.linear import Linear, linear
    torch.manual_seed(0)
    ref_layer = torch.nn.Linear(64, 48).cuda()
    m = Linear.from_linear(ref_layer)
    x = torch.randn(500, 64, device="cuda", requires_grad=True)
    y = m(x)
    y_ref = ref_layer(x.detach())
    assert torch.allclose(y.detach(), y_ref.detach(), rtol=1e-5, atol=1e-5)
    y.sum().backward()
    assert torch.allclose(x.grad, ref_layer.weight.detach().sum(0).expand(500, 64), rtol=1e-5, atol=1e-5)
    w = torch.randn(48, 64, device="cuda", requires_grad=True)
    with pytest.raises(RuntimeError, match="input gradient only"):
        linear(torch.randn(5, 64, device="cuda", requires_grad=True), w).sum().backward()
    # weight changes are picked up (planes re-split)
    with torch.no_grad():
        m.weight.mul_(2.0)
    y2 = m(x.detach())
    assert torch.allclose(y2, 2.0 * (y.detach() - m.bias) + m.bias, rtol=1e-5, atol=1e-5)


def test_converted_model_forward_and_input_gradient(fe):
    """A small MLP converted by convert_linears: the same outputs and input
    gradients as the FP32 torch model (to FP32 accuracy), with and without the
    fused GELU."""
    from fp32_emulated_gemm_amd.linear import Linear, convert_linears
    torch.manual_seed(11)

    def mlp():
        torch.manual_seed(11)
        return torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(), torch.nn.Linear(256, 64)).cuda()

    ref = mlp()
    x = torch.randn(1200, 64, device="cuda")
    xr = x.clone().requires_grad_(True)
    y_ref = ref(xr)
    y_ref.sum().backward()
    m = convert_linears(mlp())
    assert isinstance(m[0], Linear) and isinstance(m[2], Linear)
    xe = x.clone().requires_grad_(True)
    y = m(xe)
    y.sum().backward()
    assert torch.allclose(y.detach(), y_ref.detach(), rtol=1e-5, atol=1e-5)
    assert torch.allclose(xe.grad, xr.grad, rtol=1e-4, atol=1e-5)
    f = convert_linears(mlp(), fuse_gelu=True)
    assert f[0].activation == "gelu" and isinstance(f[1], torch.nn.Identity)
    with torch.no_grad():
        yf = f(x)
    assert torch.allclose(yf, y_ref.detach(), rtol=1e-5, atol=1e-5)
