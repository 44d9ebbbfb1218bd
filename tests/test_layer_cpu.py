"""Host-side checks of the torch layer: argument validation happens before any
GPU call, and there is no CPU path (CPU tensors raise)."""
import pytest
import torch

from deterministic_invariant_gemm_amd.torch_layer import Linear, deterministic_linear


def test_cpu_tensors_raise():
    x, w = torch.zeros(4, 8, dtype=torch.bfloat16), torch.zeros(8, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        deterministic_linear(x, w)


def test_shape_and_dtype_validation():
    w = torch.zeros(8, 16)
    with pytest.raises(ValueError, match="does not match"):
        deterministic_linear(torch.zeros(4, 9), w)
    with pytest.raises(ValueError, match=r"\[in, out\]"):
        deterministic_linear(torch.zeros(4, 8), torch.zeros(8))
    with pytest.raises(ValueError, match="bias"):
        deterministic_linear(torch.zeros(4, 8), w, torch.zeros(15))


def test_linear_stores_weight_in_out_and_from_torch_transposes():
    torch.manual_seed(0)
    ref = torch.nn.Linear(5, 7)
    lay = Linear.from_torch(ref)
    assert lay.weight.shape == (5, 7)
    assert torch.equal(lay.weight, ref.weight.t())
    assert torch.equal(lay.bias, ref.bias)
    fresh = Linear(10, 3, bias=False)
    assert fresh.bias is None and fresh.weight.shape == (10, 3)
    assert float(fresh.weight.detach().abs().max()) <= 1 / 10 ** 0.5
