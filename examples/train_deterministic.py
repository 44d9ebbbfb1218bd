"""Train a small two-layer MLP twice from one seed and check that the final
weights are bit-identical, then check batch invariance of the trained model
(sgemm-bi PyPI page: the training example trains twice and compares the
weights bit for bit, then checks that a row's output does not depend on the
rest of the batch).

Every linear layer (forward, input, weight and bias gradients) runs in this
library's HIP kernels; the ReLU, the mean-squared-error loss and the SGD update
are plain elementwise torch operations.  Data are seeded synthetic Gaussians.

    python examples/train_deterministic.py [--steps 20] [--dtype bf16]
"""
from __future__ import annotations

import argparse
import hashlib
import os
import sys

import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from deterministic_invariant_gemm_amd.torch_layer import Linear  # noqa: E402

DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def make_model(d_in, d_hidden, d_out, dtype, seed):
    torch.manual_seed(seed)  # CPU generator: same initial weights every time
    model = torch.nn.Sequential(Linear(d_in, d_hidden, dtype=dtype), torch.nn.ReLU(),
                                Linear(d_hidden, d_out, dtype=dtype))
    return model.cuda()


def train(seed=0, steps=20, batch=512, d_in=768, d_hidden=3072, d_out=768, dtype=torch.bfloat16,
          lr=0.05):
    """Run `steps` SGD steps; return the model and the per-step losses."""
    model = make_model(d_in, d_hidden, d_out, dtype, seed)
    g = torch.Generator().manual_seed(seed + 1)
    teacher = torch.randn(d_in, d_out, generator=g) / d_in ** 0.5
    losses = []
    for _ in range(steps):
        x = torch.randn(batch, d_in, generator=g)
        t = torch.tanh(x @ teacher)
        x, t = x.to(dtype).cuda(), t.cuda()
        y = model(x)
        loss = (y.float() - t).pow(2).mean()
        model.zero_grad(set_to_none=True)
        loss.backward()
        with torch.no_grad():
            for p in model.parameters():
                p.sub_(lr * p.grad)
        losses.append(float(loss.detach()))
    return model, losses


def digest(model) -> str:
    h = hashlib.sha256()
    for p in model.parameters():
        h.update(p.detach().contiguous().view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()


def batch_invariant(model, d_in, dtype, rows=(1, 3, 17, 128), seed=7) -> bool:
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(max(rows) * 4, d_in, generator=g).to(dtype).cuda()
    with torch.no_grad():
        full = model(x)
        return all(torch.equal(model(x[:r]), full[:r]) for r in rows)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--batch", type=int, default=512)
    ap.add_argument("--dtype", choices=sorted(DTYPES), default="bf16")
    ap.add_argument("--seed", type=int, default=0)
    a = ap.parse_args(argv)
    dtype = DTYPES[a.dtype]
    m1, l1 = train(a.seed, a.steps, a.batch, dtype=dtype)
    m2, l2 = train(a.seed, a.steps, a.batch, dtype=dtype)
    d1, d2 = digest(m1), digest(m2)
    same = d1 == d2 and l1 == l2
    inv = batch_invariant(m1, 768, dtype)
    print(f"loss {l1[0]:.5f} -> {l1[-1]:.5f} over {a.steps} steps")
    print(f"weights run 1 {d1[:16]}  run 2 {d2[:16]}  bit-identical: {same}")
    print(f"batch-invariant forward after training: {inv}")
    return 0 if same and inv else 1


if __name__ == "__main__":
    sys.exit(main())
