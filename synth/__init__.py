"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and converts them to the storage formats; it
holds none of the GEMM arithmetic.  Both the CPU oracle and the HIP path consume
exactly the arrays produced here.

Recipe: every tensor ``idx`` of a workload with seed ``seed`` is drawn from
``numpy.random.Generator(PCG64(seed * 1000 + idx)).standard_normal`` in float64,
multiplied by sigma, cast to float32 and then rounded to the storage dtype with
torch's CPU cast (round-to-nearest-even).  Arrays are returned as bit patterns:
uint32 for f32, uint16 for bf16 / f16, uint8 for fp8 e4m3fn codes.
"""
from __future__ import annotations

import numpy as np
import torch

F32, BF16, F16 = 0, 1, 2
NAMES = {F32: "f32", BF16: "bf16", F16: "f16"}
_TORCH = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}
STORAGE = {F32: np.uint32, BF16: np.uint16, F16: np.uint16}
PAD_ID = 0xFFFFFFFF


def rng(seed: int, idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed * 1000 + idx))


def normal_f32(shape, sigma: float, seed: int, idx: int) -> np.ndarray:
    return (rng(seed, idx).standard_normal(shape) * sigma).astype(np.float32)


def to_bits(a: np.ndarray, dt: int) -> np.ndarray:
    """float32 array -> bit patterns of dtype dt (RNE via torch's CPU cast)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dt == F32:
        return a.view(np.uint32).copy()
    t = torch.from_numpy(a).to(_TORCH[dt])
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f32(bits: np.ndarray, dt: int) -> np.ndarray:
    """bit patterns of dtype dt -> float32 values (exact widening)."""
    if dt == F32:
        return np.ascontiguousarray(bits).view(np.float32)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(_TORCH[dt])
    return t.to(torch.float32).numpy()


def normal_bits(shape, sigma, seed, idx, dt):
    return to_bits(normal_f32(shape, sigma, seed, idx), dt)


def integer_bits(shape, lo, hi, seed, idx, dt):
    """Uniform integers in [lo, hi] stored exactly in dtype dt."""
    v = rng(seed, idx).integers(lo, hi + 1, size=shape).astype(np.float32)
    return to_bits(v, dt)


def wide_exponent_bits(shape, dt, seed, idx, emin, emax):
    """Values sign * 2^e * (1 + f) with e uniform in [emin, emax] and f a
    uniformly drawn fraction of the dtype's significand width, so every value
    is exact in dt (products of two such values span many binades)."""
    frac_bits = {BF16: 7, F16: 10, F32: 23}[dt]
    g = rng(seed, idx)
    sign = np.where(g.integers(0, 2, size=shape) == 1, -1.0, 1.0)
    e = g.integers(emin, emax + 1, size=shape).astype(np.float64)
    f = g.integers(0, 1 << frac_bits, size=shape).astype(np.float64) / (1 << frac_bits)
    return to_bits((sign * np.exp2(e) * (1.0 + f)).astype(np.float32), dt)


def hashed_ints(rows, cols, lo, hi, seed, idx, xp=np, device=None):
    """Integers in [lo, hi] at (r, c) for r in ``rows``, c in ``cols`` (index
    arrays), from a closed-form 32-bit hash of (r, c, seed, idx), as float32 --
    so any block of a very large tensor can be produced on its own, by numpy
    (``xp=np``) or by torch on a device (``xp=torch``), with the same values.
    Every row differs from every other with high probability, so a row or
    column index off by any amount changes the values read."""
    if xp is np:
        r = np.asarray(rows, dtype=np.int64)[:, None]
        c = np.asarray(cols, dtype=np.int64)[None, :]
    else:
        r = torch.as_tensor(rows, dtype=torch.int64, device=device)[:, None]
        c = torch.as_tensor(cols, dtype=torch.int64, device=device)[None, :]
    m32 = 0xFFFFFFFF
    h = (r * 0x9E3779B1 + c * 0x85EBCA77 + (seed * 1000 + idx) * 0xC2B2AE3D) & m32
    h = h ^ (h >> 15)
    h = (h * 0x2C1B3C6D) & m32
    h = h ^ (h >> 12)
    v = lo + h % (hi - lo + 1)
    return v.astype(np.float32) if xp is np else v.to(torch.float32)


# --------------------------------------------------------------------------
# linear workloads
# --------------------------------------------------------------------------

def linear(m, k, n, dt, seed, sigma_x=1.0, sigma_w=1.0, sigma_b=1.0, sigma_dy=1.0,
           bias=True):
    """X[m,k], W[k,n] (stored [in,out]), b[n], dY[m,n]."""
    return {
        "x": normal_bits((m, k), sigma_x, seed, 0, dt),
        "w": normal_bits((k, n), sigma_w, seed, 1, dt),
        "b": normal_bits((n,), sigma_b, seed, 2, dt) if bias else None,
        "dy": normal_bits((m, n), sigma_dy, seed, 3, dt),
        "m": m, "k": k, "n": n, "dt": dt,
    }


def linear_integer(m, k, n, dt, seed, lo=-4, hi=4, bias=True):
    """Small-integer operands: every partial sum stays an integer below 2^24
    in magnitude (for K, N, M up to about 10^6 / 16), so f32 accumulation is
    exact in any order."""
    return {
        "x": integer_bits((m, k), lo, hi, seed, 0, dt),
        "w": integer_bits((k, n), lo, hi, seed, 1, dt),
        "b": integer_bits((n,), lo, hi, seed, 2, dt) if bias else None,
        "dy": integer_bits((m, n), lo, hi, seed, 3, dt),
        "m": m, "k": k, "n": n, "dt": dt,
    }


def f32_linear_64x128x256():
    """f32 X[64,128], W[128,256], b[256], dY[64,256], all N(0,1)."""
    return linear(64, 128, 256, F32, seed=1)


def mlp_up_linear(dt=BF16, n=3072, seed=2):
    """Transformer MLP-up linear 768 -> 3072 at M=4096: X, dY ~ N(0,1);
    W, b ~ N(0,0.02).  dt=F16 gives the f16 rerun from the same f32 draws;
    n=48, seed=22 gives the narrow-output case."""
    return linear(4096, 768, n, dt, seed, sigma_x=1.0, sigma_w=0.02, sigma_b=0.02,
                  sigma_dy=1.0)


def square_4096_sweep():
    """Batch-invariance sweep: W[4096,4096] ~ N(0,0.02), X[8192,4096] and
    dY[8192,4096] ~ N(0,1), no bias."""
    return linear(8192, 4096, 4096, BF16, seed=3, sigma_w=0.02, bias=False)


# --------------------------------------------------------------------------
# fp8 workload
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def quantize_e4m3(bf16_bits: np.ndarray):
    """Per-tensor quantisation used to prepare fp8 inputs: amax over the
    tensor, scale s = 448 / amax (f32), codes = e4m3fn(clamp(x * s, +-448)) by
    torch's RNE cast; returns (codes uint8, dequant scale f32(1/s))."""
    x = torch.from_numpy(to_f32(bf16_bits, BF16))
    amax = float(x.abs().max())
    s = np.float32(E4M3_MAX / amax) if amax > 0 else np.float32(1.0)
    q = (x * float(s)).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    codes = q.view(torch.uint8).numpy().copy()
    return codes, np.float32(1.0 / np.float64(s))


def fp8(m, k, n, seed):
    a = normal_bits((m, k), 1.0, seed, 0, BF16)
    bt = normal_bits((n, k), 1.0, seed, 1, BF16)
    a8, da = quantize_e4m3(a)
    b8, db = quantize_e4m3(bt)
    return {"a8": a8, "bt8": b8, "da": da, "db": db, "m": m, "k": k, "n": n}


def fp8_linear(m, k, n, seed, sigma_w=0.02, bias=True):
    """bf16 operands of the scaled fp8 linear: x [m,k] ~ N(0,1), w [n,k]
    ([out,in]) ~ N(0, sigma_w), bias [n] ~ N(0, 0.02), g [m,n] ~ N(0,1), and
    per-tensor scales from each tensor's max-abs (delayed-scaling style:
    scale = amax / 448 as an f32, scale_inv = 448 / amax)."""
    x = normal_bits((m, k), 1.0, seed, 0, BF16)
    w = normal_bits((n, k), sigma_w, seed, 1, BF16)
    g = normal_bits((m, n), 1.0, seed, 3, BF16)
    b = normal_bits((n,), 0.02, seed, 2, BF16) if bias else None
    out = {"x": x, "w": w, "g": g, "b": b, "m": m, "k": k, "n": n}
    for name in ("x", "w", "g"):
        amax = float(np.abs(to_f32(out[name], BF16)).max()) if out[name].size else 1.0
        amax = amax if amax > 0 else 1.0
        out["s" + name] = np.float32(amax / E4M3_MAX)
        out["s" + name + "_inv"] = np.float32(E4M3_MAX / amax)
    return out


def fp8_8192x4096x4096():
    """fp8 e4m3: A[8192,4096], B^T[4096,4096] from N(0,1) bf16."""
    return fp8(8192, 4096, 4096, seed=4)


def fp8_integer(m, k, n, seed, lo=-8, hi=8, da=0.5, db=0.25):
    """Small-integer e4m3 codes with power-of-two scales: exact in any order."""
    a = torch.from_numpy(rng(seed, 0).integers(lo, hi + 1, size=(m, k)).astype(np.float32))
    b = torch.from_numpy(rng(seed, 1).integers(lo, hi + 1, size=(n, k)).astype(np.float32))
    return {"a8": a.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy(),
            "bt8": b.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy(),
            "da": np.float32(da), "db": np.float32(db), "m": m, "k": k, "n": n}


# --------------------------------------------------------------------------
# grouped workload
# --------------------------------------------------------------------------

def route(m, e, seed, pad_rows=0, empty=(), idx=9):
    """Row routing: ids uniform over [0,e) (experts listed in `empty` receive
    no rows), `pad_rows` rows set to 0xFFFFFFFF chosen by a seeded permutation,
    then sorted ascending (padding last).  offsets[j] = number of rows whose id
    is below j, for j = 0..e."""
    g = rng(seed, idx)
    allowed = np.array([j for j in range(e) if j not in set(empty)], dtype=np.int64)
    ids = allowed[g.integers(0, len(allowed), size=m)].astype(np.uint32) if len(allowed) \
        else np.full(m, PAD_ID, dtype=np.uint32)
    if pad_rows:
        ids[g.permutation(m)[:pad_rows]] = PAD_ID
    ids = np.sort(ids, kind="stable").astype(np.uint32)
    offsets = np.array([np.count_nonzero(ids < j) for j in range(e + 1)], dtype=np.uint32)
    return ids, offsets


def grouped(m, k, n, e, dt, seed, pad_rows=0, empty=(), sigma_w=0.02):
    ids, offsets = route(m, e, seed, pad_rows, empty)
    return {
        "input": normal_bits((m, k), 1.0, seed, 0, dt),
        "weights": normal_bits((e, n, k), sigma_w, seed, 1, dt),
        "dy": normal_bits((m, n), 1.0, seed, 3, dt),
        "row_experts": ids, "offsets": offsets,
        "m": m, "k": k, "n": n, "e": e, "dt": dt,
    }


def grouped_16384x2048x1408_e8(empty=()):
    """input[16384,2048] ~ N(0,1), weights[8,1408,2048] ~ N(0,0.02), 5 % of
    rows (819) padding, dY[16384,1408] ~ N(0,1)."""
    return grouped(16384, 2048, 1408, 8, BF16, seed=5, pad_rows=round(0.05 * 16384),
                   empty=empty)
