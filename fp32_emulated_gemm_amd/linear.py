"""Linear layer on the BF16x9 emulated SGEMM (a thin torch op over the C ABI).

The pages use the emulation as a drop-in for the FP32 matrix multiplication of
the linear layers of an interatomic potential, keeping the trained weights and
layer shapes (NVIDIA Technical Blog, "Unlocking Tensor Core Performance for
Machine Learning Interatomic Potentials", section "TF32x3 on NVIDIA Ampere
GPUs"; discuss.pytorch.kr summary, section "PyTorch에서 직접 써 보려면").
Forces are gradients of the energy with respect to the inputs, so the layer
provides the forward product and the input gradient, both emulated:

    forward   Y  = X W^T + b      sgemm_emu_linear (W's planes, N x K)
    backward  dX = dY W           sgemm_emu_presplit_b (the planes of W^T, N x K)

The weight [out_features][in_features] is split once into the planes of W and
of W^T (the N x K layout is the one the GEMM copies straight into LDS for both
products) and reused until the weight tensor changes.  Parameter gradients (dW, db)
are not provided: the layer is for fixed weights, its parameters are created
with requires_grad=False, and a backward pass that would need them raises.
"""
import torch

from . import (SGEMM_EMU_ACT_GELU, SGEMM_EMU_ACT_NONE, SGEMM_EMU_B_NK, sgemm_emu_linear, sgemm_emu_presplit_b, split,
               split_t)

_ACTIVATIONS = {None: SGEMM_EMU_ACT_NONE, "gelu": SGEMM_EMU_ACT_GELU}


def split_weight(weight):
    """(planes of W [out][in], planes of W^T [in][out]) for the forward product
    and the input gradient."""
    w = weight.detach().contiguous()
    return split(w), split_t(w)


class WeightPlanes:
    """split_weight of a [out][in] weight, redone when the weight changes."""

    def __init__(self):
        self._key = None
        self.planes = None

    def get(self, weight):
        key = (weight.data_ptr(), weight._version, tuple(weight.shape), weight.device)
        if key != self._key:
            self.planes = split_weight(weight)
            self._key = key
        return self.planes


class _LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x2d, weight, bias, planes, nbands, act):
        M, K = x2d.shape
        N = weight.shape[0]
        y = torch.empty((M, N), dtype=torch.float32, device=x2d.device)
        w0, w1, w2 = planes[0]
        sgemm_emu_linear(M, N, K, x2d, max(K, 1), w0, w1, w2, max(K, 1), bias, act, y, max(N, 1), nbands)
        ctx.planes = planes[1]
        ctx.nbands = nbands
        ctx.shape = (M, N, K)
        return y

    @staticmethod
    def backward(ctx, dy):
        if ctx.needs_input_grad[1] or ctx.needs_input_grad[2]:
            raise RuntimeError("fp32_emulated_gemm_amd.linear provides the input gradient only; "
                               "set requires_grad=False on the weight and bias")
        M, N, K = ctx.shape
        t0, t1, t2 = ctx.planes             # W^T: K x N of the backward product dY[M x N] W[N x K]
        dy = dy.contiguous()
        dx = torch.empty((M, K), dtype=torch.float32, device=dy.device)
        sgemm_emu_presplit_b(M, K, N, dy, max(N, 1), t0, t1, t2, max(N, 1), SGEMM_EMU_B_NK, dx, max(K, 1),
                             ctx.nbands)
        return dx, None, None, None, None, None


def linear(x, weight, bias=None, nbands=5, planes=None, activation=None):
    """Y = act(x W^T + b) on the emulated GEMM, for float32 CUDA tensors x[..., in],
    weight[out, in], bias[out]; activation None or "gelu" (exact erf form, fused
    into the GEMM's epilogue, forward only).  `planes` (from
    `split_weight(weight)`) skips the split."""
    if x.dtype != torch.float32 or weight.dtype != torch.float32:
        raise TypeError("linear expects float32 tensors")
    if activation not in _ACTIVATIONS:
        raise ValueError(f"unknown activation {activation!r}")
    act = _ACTIVATIONS[activation]
    if act != SGEMM_EMU_ACT_NONE and torch.is_grad_enabled() and x.requires_grad:
        raise NotImplementedError("the fused activation runs forward only; apply it separately to differentiate")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (weight.shape[0],)):
        raise ValueError("bias must be float32 of shape [out_features]")
    if planes is None:
        planes = split_weight(weight)
    lead = x.shape[:-1]
    x2d = x.reshape(-1, x.shape[-1]).contiguous()
    b = None if bias is None else bias.contiguous()
    y = _LinearFn.apply(x2d, weight, b, planes, nbands, act)
    return y.reshape(*lead, weight.shape[0])


class Linear(torch.nn.Module):
    """Drop-in for torch.nn.Linear (fixed weights) running on the emulated GEMM."""

    def __init__(self, in_features, out_features, bias=True, nbands=5, device=None, activation=None):
        super().__init__()
        self.in_features, self.out_features, self.nbands = in_features, out_features, nbands
        self.activation = activation
        self.weight = torch.nn.Parameter(torch.empty((out_features, in_features), device=device),
                                         requires_grad=False)
        self.bias = (torch.nn.Parameter(torch.zeros(out_features, device=device), requires_grad=False)
                     if bias else None)
        self._planes = WeightPlanes()

    @classmethod
    def from_linear(cls, layer, nbands=5):
        m = cls(layer.in_features, layer.out_features, layer.bias is not None, nbands, layer.weight.device)
        with torch.no_grad():
            m.weight.copy_(layer.weight)
            if layer.bias is not None:
                m.bias.copy_(layer.bias)
        return m

    def forward(self, x):
        return linear(x, self.weight, self.bias, self.nbands, self._planes.get(self.weight), self.activation)

    def extra_repr(self):
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, nbands={self.nbands}, activation={self.activation}")


def convert_linears(module, nbands=5, fuse_gelu=False):
    """Swap every torch.nn.Linear inside `module` (recursively, in place) for a
    Linear holding the same weights: the fixed-weight use in which the pages
    replace a model's FP32 layers by an emulated-GEMM layer with its trained
    weights and shapes unchanged.  Returns `module`, or its replacement when
    `module` is itself an nn.Linear.

    fuse_gelu: inside nn.Sequential containers, an nn.Linear directly followed
    by nn.GELU (the exact erf form) becomes one Linear with the GELU applied in
    the GEMM's epilogue, and the GELU module an nn.Identity.  The fused
    activation is forward-only (no input gradient), so leave it off where
    gradients with respect to the inputs are needed (forces)."""
    if isinstance(module, torch.nn.Linear):
        return Linear.from_linear(module, nbands)
    children = list(module.named_children())
    for i, (name, child) in enumerate(children):
        new = convert_linears(child, nbands, fuse_gelu)
        if new is not child:
            setattr(module, name, new)
        if (fuse_gelu and isinstance(module, torch.nn.Sequential) and isinstance(child, torch.nn.Linear)
                and i + 1 < len(children) and isinstance(children[i + 1][1], torch.nn.GELU)
                and children[i + 1][1].approximate == "none"):
            new.activation = "gelu"
            setattr(module, children[i + 1][0], torch.nn.Identity())
    return module
