"""Helpers shared by the GPU parity tests: device buffers from host bit arrays,
the per-element pass rule against the oracle, hashing and run-to-run checks.

Pass rule (per output element, given the oracle's exact pre-rounding value S
and absolute-product scale A):
  * f32 outputs:      |gpu - S| <= 1e-5 * A
  * bf16/f16 outputs: ulp distance between the GPU bits and RNE(S) <= 1, or
                      |gpu - S| <= 1e-5 * A  (near-cancellation elements, where
                      the f32 accumulation error the contract allows exceeds
                      one ulp of the small result)
  * never NaN where the oracle is finite.
The fp8 GEMMs' opt-in fast path (tc = 3) alone is checked with the wider rule
check(..., groups=True): 2^-10 * G is added to the second clause, G = sum over
groups of 8 consecutive reduction indices of the largest |product| (the
oracle's .g), because the fp8 matrix instruction adds each such group aligned
to its largest product with 13 bits below it (measured on gfx950,
test_fp8_fast_group_alignment), so each product may lose up to 2^-13 of its
group's maximum.  The default fp8 path meets the plain rule.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

import synth

REL = 1e-5

_TORCH_BITS = {np.dtype(np.uint16): torch.int16, np.dtype(np.uint32): torch.int32,
               np.dtype(np.uint8): torch.uint8}


def dev(bits: np.ndarray) -> torch.Tensor:
    """Copy a host bit-pattern array to the GPU (same bytes, integer view)."""
    a = np.ascontiguousarray(bits)
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32,
            np.dtype(np.uint8): np.uint8}[a.dtype]
    return torch.from_numpy(a.view(view).copy()).cuda()


def empty(shape, storage) -> torch.Tensor:
    """Poisoned output buffer (all bits 1) of the given numpy storage dtype."""
    t = torch.empty(shape, dtype=_TORCH_BITS[np.dtype(storage)], device="cuda")
    t.fill_(-1 if storage != np.uint8 else 255)
    return t


def host(t: torch.Tensor, storage) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy().view(storage)


def f32_scalar(v: float) -> torch.Tensor:
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def digest(t: torch.Tensor) -> str:
    torch.cuda.synchronize()
    return hashlib.sha256(t.cpu().numpy().tobytes()).hexdigest()


def ord16(bits: np.ndarray) -> np.ndarray:
    """Monotone integer image of bf16/f16 bit patterns (+0 and -0 map to 0)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def decode(bits: np.ndarray, dt: int) -> np.ndarray:
    return synth.to_f32(np.ascontiguousarray(bits), dt).astype(np.float64)


def check(gpu_bits: np.ndarray, res, dt: int, what: str = "", rel: float = REL,
          groups: bool = False):
    """Assert the pass rule (with groups=True the fp8 fast path's wider one);
    return (max ulp, #elements beyond 1 ulp, max |gpu - S| / A)."""
    gpu_bits = np.ascontiguousarray(gpu_bits).reshape(res.out.shape)
    val = decode(gpu_bits, dt)
    err = np.abs(val - res.s)
    scale = np.maximum(res.a, 1e-300)
    finite = np.isfinite(res.s)
    assert not np.any(np.isnan(val) & finite), f"{what}: NaN in GPU output"
    if dt == synth.F32:
        bad = finite & (err > rel * res.a)
        nbad = int(bad.sum())
        assert nbad == 0, (f"{what}: {nbad} f32 elements off; worst rel "
                           f"{float(np.max(err / scale)):.3g}")
        return 0, 0, float(np.max(np.where(finite, err / scale, 0)))
    ulp = np.abs(ord16(gpu_bits) - ord16(res.out))
    tol = rel * res.a
    if groups:
        # fp8 matrix instruction: each group of 8 products is added aligned to
        # its largest one, keeping 13 bits below it, so every product may lose
        # up to 2^-13 of the group maximum: at most 2^-10 per group maximum
        tol = tol + 2.0 ** -10 * res.g
    close = err <= tol
    bad = finite & (ulp > 1) & ~close
    nbad = int(bad.sum())
    if nbad:
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(i), int(gpu_bits[tuple(i)]), int(res.out[tuple(i)]),
                   float(res.s[tuple(i)]), float(res.a[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {nbad} elements beyond 1 ulp and 1e-5*A: {detail}")
    return int(ulp[finite].max(initial=0)), int(((ulp > 1) & finite).sum()), \
        float(np.max(np.where(finite, err / scale, 0)))


def sample_rows(total: int, count: int, seed: int) -> np.ndarray:
    """First, last and a seeded random spread of row indices."""
    g = np.random.default_rng(seed)
    rows = {0, total - 1, total // 2}
    rows.update(g.choice(total, size=min(count, total), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def group_stats(gpu_bits: np.ndarray, res, dt: int, rel: float = REL):
    """(max ulp, #elements beyond 1 ulp, #elements that pass only through the
    2^-10 * G clause of the fp8 fast path's rule)."""
    gpu_bits = np.ascontiguousarray(gpu_bits).reshape(res.out.shape)
    err = np.abs(decode(gpu_bits, dt) - res.s)
    finite = np.isfinite(res.s)
    ulp = np.abs(ord16(gpu_bits) - ord16(res.out))
    need_g = finite & (ulp > 1) & (err > rel * res.a)
    return int(ulp[finite].max(initial=0)), int(((ulp > 1) & finite).sum()), int(need_g.sum())
