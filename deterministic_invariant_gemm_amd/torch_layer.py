"""PyTorch layer over the C ABI: a linear layer whose forward, input gradient,
weight gradient and bias gradient all run in this library's HIP kernels.

The weight is stored ``[in, out]`` (sgemm-bi PyPI page, "Use": the layer keeps
its weight in the GEMM-natural ``[in, out]`` layout, and ``from_torch`` turns an
``nn.Linear`` into one), so ``y = x @ weight + bias`` maps directly onto
``bi_forward``.  Backward follows ViperLLM ffma.py, _FFMAAddmm.backward: the
input gradient ``gy @ weight^T`` and the weight gradient ``x^T @ gy`` returned
in the weight dtype (both from ``bi_linear_backward``, or ``bi_backward_dx`` /
``bi_backward_dw`` when only one is needed; same bits) and the bias gradient
as an f32 column sum cast back once (``bi_bias_grad``).

Torch supplies device memory, the current stream and autograd bookkeeping only.
Tensors must be CUDA (HIP) tensors of one dtype (float32, bfloat16 or float16);
anything else raises, and there is no CPU path.
"""
from __future__ import annotations

import math

import torch

from . import (BI_BF16, BI_F16, BI_F32, bi_backward_dw, bi_backward_dw_workspace_bytes,
               bi_backward_dx, bi_bias_grad, bi_bias_grad_workspace_bytes, bi_forward,
               bi_linear_backward, check)

_DTYPES = {torch.float32: BI_F32, torch.bfloat16: BI_BF16, torch.float16: BI_F16}


def _tc(tensor_cores) -> int:
    """tensor_cores: True (automatic MFMA tier), False (scalar tier) or an int
    tier request passed through unchanged (2 = MFMA required)."""
    if isinstance(tensor_cores, bool):
        return 1 if tensor_cores else 0
    return int(tensor_cores)


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _validate(x, weight, bias):
    if weight.dim() != 2:
        raise ValueError(f"weight must be [in, out], got shape {tuple(weight.shape)}")
    if x.dim() < 1 or x.shape[-1] != weight.shape[0]:
        raise ValueError(f"x [..., {x.shape[-1] if x.dim() else '?'}] does not match weight "
                         f"[in={weight.shape[0]}, out={weight.shape[1]}]")
    if bias is not None and tuple(bias.shape) != (weight.shape[1],):
        raise ValueError(f"bias must be [{weight.shape[1]}], got {tuple(bias.shape)}")
    tensors = [x, weight] + ([bias] if bias is not None else [])
    if any(not t.is_cuda for t in tensors):
        raise ValueError("deterministic_linear needs GPU tensors (no CPU path)")
    if any(t.dtype != x.dtype for t in tensors):
        raise ValueError("x, weight and bias must share one dtype")
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    if any(t.device != x.device for t in tensors):
        raise ValueError("x, weight and bias must be on one device")


class _LinearFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, bias, tc):
        _validate(x, weight, bias)
        k, n = weight.shape
        lead = x.shape[:-1]
        x2 = x.reshape(-1, k).contiguous()
        w = weight.contiguous()
        b = bias.contiguous() if bias is not None else None
        m = x2.shape[0]
        dt = _DTYPES[x.dtype]
        y = torch.empty((m, n), dtype=x.dtype, device=x.device)
        with torch.cuda.device(x.device):
            check(bi_forward(y, x2, w, b, m, k, n, dt, torch.cuda.current_stream(), tc),
                  "bi_forward")
        ctx.save_for_backward(x2, w)
        ctx.has_bias, ctx.tc, ctx.lead = bias is not None, tc, lead
        return y.reshape(*lead, n)

    @staticmethod
    def backward(ctx, gy):
        x2, w = ctx.saved_tensors
        k, n = w.shape
        m = x2.shape[0]
        dt = _DTYPES[w.dtype]
        gy2 = gy.to(w.dtype).reshape(-1, n).contiguous()
        dx = dw = db = None
        with torch.cuda.device(w.device):
            stream = torch.cuda.current_stream()
            if ctx.needs_input_grad[0]:
                dx = torch.empty((m, k), dtype=w.dtype, device=w.device)
            if ctx.needs_input_grad[1]:
                dw = torch.empty((k, n), dtype=w.dtype, device=w.device)
            if dx is not None and dw is not None:
                # both from one call: the library may run their tiles in one launch
                nb = bi_backward_dw_workspace_bytes(m, k, n, dt, ctx.tc)
                ws = _workspace(nb, w.device)
                check(bi_linear_backward(dx, dw, gy2, x2, w, m, k, n, dt, ws, nb, stream, ctx.tc),
                      "bi_linear_backward")
            elif dx is not None:
                check(bi_backward_dx(dx, gy2, w, m, k, n, dt, stream, ctx.tc), "bi_backward_dx")
            elif dw is not None:
                nb = bi_backward_dw_workspace_bytes(m, k, n, dt, ctx.tc)
                ws = _workspace(nb, w.device)
                check(bi_backward_dw(dw, x2, gy2, m, k, n, dt, ws, nb, stream, ctx.tc),
                      "bi_backward_dw")
            if dx is not None:
                dx = dx.reshape(*ctx.lead, k)
            if ctx.has_bias and ctx.needs_input_grad[2]:
                db = torch.empty((n,), dtype=w.dtype, device=w.device)
                nb = bi_bias_grad_workspace_bytes(m, n, dt)
                ws = _workspace(nb, w.device)
                check(bi_bias_grad(db, gy2, m, n, dt, ws, nb, stream), "bi_bias_grad")
        return dx, dw, db, None


def deterministic_linear(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None = None,
                         tensor_cores=True) -> torch.Tensor:
    """y = x @ weight + bias with weight ``[in, out]``; differentiable in all
    three.  Batch-invariant in the rows of x; bit-identical run to run."""
    return _LinearFunction.apply(x, weight, bias, _tc(tensor_cores))


class Linear(torch.nn.Module):
    """Linear layer with weight ``[in_features, out_features]``.

    Initialisation matches ``torch.nn.Linear`` (uniform in +-1/sqrt(in)) in
    distribution; use ``from_torch`` to take over an existing layer's values.
    """

    def __init__(self, in_features: int, out_features: int, bias: bool = True,
                 tensor_cores=True, device=None, dtype=None):
        super().__init__()
        self.in_features, self.out_features = in_features, out_features
        self.tensor_cores = tensor_cores
        kw = {"device": device, "dtype": dtype}
        self.weight = torch.nn.Parameter(torch.empty((in_features, out_features), **kw))
        self.bias = torch.nn.Parameter(torch.empty(out_features, **kw)) if bias else None
        self.reset_parameters()

    def reset_parameters(self):
        bound = 1.0 / math.sqrt(self.in_features) if self.in_features > 0 else 0.0
        with torch.no_grad():
            self.weight.uniform_(-bound, bound)
            if self.bias is not None:
                self.bias.uniform_(-bound, bound)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return deterministic_linear(x, self.weight, self.bias, self.tensor_cores)

    @classmethod
    def from_torch(cls, layer: torch.nn.Linear, tensor_cores=True) -> "Linear":
        """Copy of an ``nn.Linear`` (weight ``[out, in]``) with the weight
        transposed into ``[in, out]``; same device and dtype."""
        w = layer.weight
        out = cls(layer.in_features, layer.out_features, layer.bias is not None, tensor_cores,
                  device=w.device, dtype=w.dtype)
        with torch.no_grad():
            out.weight.copy_(w.detach().t())
            if layer.bias is not None:
                out.bias.copy_(layer.bias.detach())
        return out

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, tensor_cores={self.tensor_cores}")
