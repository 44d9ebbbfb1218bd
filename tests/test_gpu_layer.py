"""The torch layer over the C ABI: its forward and all three gradients against
the oracle (leading batch dims flattened), Linear.from_torch against
nn.Linear, and the train-twice example (bit-identical weights, then batch
invariance of the trained model)."""
import importlib.util
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from deterministic_invariant_gemm_amd.torch_layer import Linear, deterministic_linear
from parity import check, dev

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TORCH = {synth.F32: torch.float32, synth.BF16: torch.bfloat16, synth.F16: torch.float16}
ST = {synth.F32: np.uint32, synth.BF16: np.uint16, synth.F16: np.uint16}


def as_float(bits, dt):
    return dev(bits).view(TORCH[dt])


def bits(t, dt):
    torch.cuda.synchronize()
    return t.detach().contiguous().cpu().view(torch.int32 if dt == synth.F32 else torch.int16) \
        .numpy().view(ST[dt])


@pytest.mark.parametrize("dt", [synth.BF16, synth.F16, synth.F32])
@pytest.mark.parametrize("tc", [1, 0])
def test_layer_forward_and_gradients_match_oracle(dt, tc):
    lead, k, n = (3, 100), 200, 136
    m = lead[0] * lead[1]
    d = synth.linear(m, k, n, dt, seed=41, sigma_w=0.05)
    x = as_float(d["x"], dt).reshape(*lead, k).requires_grad_(True)
    w = as_float(d["w"], dt).requires_grad_(True)
    b = as_float(d["b"], dt).requires_grad_(True)
    print(f"layer dt={dt} tc={tc}", flush=True)
    y = deterministic_linear(x, w, b, tensor_cores=bool(tc))
    assert y.shape == (*lead, n) and y.dtype == TORCH[dt]
    check(bits(y, dt), oracle.linear_forward(dt, d["x"], d["w"], d["b"], m, k, n), dt, "fwd")
    y.backward(as_float(d["dy"], dt).reshape(*lead, n))
    check(bits(x.grad.reshape(m, k), dt), oracle.linear_dx(dt, d["dy"], d["w"], m, k, n), dt, "dX")
    check(bits(w.grad, dt), oracle.linear_dw(dt, d["x"], d["dy"], m, k, n), dt, "dW")
    check(bits(b.grad, dt), oracle.bias_grad(dt, d["dy"], m, n), dt, "db")


def test_layer_without_bias_and_frozen_input():
    m, k, n, dt = 257, 128, 192, synth.BF16
    d = synth.linear(m, k, n, dt, seed=42, bias=False)
    x = as_float(d["x"], dt)  # no grad wanted for x
    w = as_float(d["w"], dt).requires_grad_(True)
    y = deterministic_linear(x, w)
    y.backward(as_float(d["dy"], dt))
    check(bits(w.grad, dt), oracle.linear_dw(dt, d["x"], d["dy"], m, k, n), dt, "dW")


def test_from_torch_matches_nn_linear():
    torch.manual_seed(3)
    ref = torch.nn.Linear(256, 320).to(torch.bfloat16).cuda()
    lay = Linear.from_torch(ref)
    assert torch.equal(lay.weight, ref.weight.t())
    assert torch.equal(lay.bias, ref.bias)
    x = torch.randn(64, 256, dtype=torch.bfloat16, device="cuda")
    y = lay(x).detach()
    # f32 reference on the CPU, one bf16 rounding apart at most (plus f32 order)
    w32, b32 = ref.weight.detach().float().cpu(), ref.bias.detach().float().cpu()
    y32 = x.float().cpu() @ w32.t() + b32
    err = (y.float().cpu() - y32).abs()
    assert float((err / (y32.abs() + 1e-2)).max()) < 2 ** -7


def test_layer_rejects_cpu_and_mixed_dtypes():
    w = torch.zeros(8, 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        deterministic_linear(torch.zeros(2, 8, dtype=torch.float16, device="cuda"), w)


def test_train_twice_example():
    spec = importlib.util.spec_from_file_location(
        "train_deterministic", os.path.join(ROOT, "examples", "train_deterministic.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert mod.main(["--steps", "6", "--batch", "256"]) == 0
