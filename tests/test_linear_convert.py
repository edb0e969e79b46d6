"""convert_linears on the CPU: which modules are swapped, that the weights are
carried over, and the optional GELU fusion (no forward pass: that needs a GPU,
see tests/test_gpu_linear.py)."""
import torch

from fp32_emulated_gemm_amd.linear import Linear, convert_linears


def _mlp():
    torch.manual_seed(3)
    return torch.nn.Sequential(torch.nn.Linear(16, 32), torch.nn.GELU(), torch.nn.Linear(32, 8, bias=False),
                               torch.nn.Sequential(torch.nn.Linear(8, 8), torch.nn.GELU(approximate="tanh")))


def test_swaps_every_linear_and_keeps_weights():
    ref = _mlp()
    m = convert_linears(_mlp())
    assert isinstance(m[0], Linear) and isinstance(m[2], Linear) and isinstance(m[3][0], Linear)
    assert isinstance(m[1], torch.nn.GELU) and isinstance(m[3][1], torch.nn.GELU)
    for a, b in ((m[0], ref[0]), (m[2], ref[2]), (m[3][0], ref[3][0])):
        assert torch.equal(a.weight, b.weight) and not a.weight.requires_grad
        assert (a.bias is None) == (b.bias is None)
        if a.bias is not None:
            assert torch.equal(a.bias, b.bias)
        assert a.activation is None and a.nbands == 5


def test_top_level_linear_and_nbands():
    lin = torch.nn.Linear(4, 3)
    m = convert_linears(lin, nbands=2)
    assert isinstance(m, Linear) and m.nbands == 2 and m is not lin


def test_fuse_gelu_only_exact_form():
    m = convert_linears(_mlp(), fuse_gelu=True)
    assert m[0].activation == "gelu" and isinstance(m[1], torch.nn.Identity)
    assert m[2].activation is None
    assert m[3][0].activation is None and isinstance(m[3][1], torch.nn.GELU)   # tanh form left alone
