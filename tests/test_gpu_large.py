"""Operands and outputs beyond 4 GiB.

X [524288, 4608] bf16 is 4.8 GB: the forward and dW read it through the
register-staged MFMA kernel (the direct-load kernel addresses its operands with
32-bit buffer offsets and takes operands up to 1 GiB), and dX writes a 4.8 GB
output.  Inputs are small integers from a closed-form hash (generated on the GPU
block by block, and on the host for the sampled rows and columns), so every sum
is exact in f32 and the GPU bits must equal the oracle's exactly.  Sampled rows
and columns include ones whose byte offsets lie beyond 2^32.  The fp8 GEMM is
checked the same way on A [1048576, 4608] e4m3 (4.8 GB, register-staged fp8
kernel), the grouped forward on X, and the f32 scalar tier on X f32
[524288, 2304] (4.8 GB).
"""
import numpy as np
import pytest
import torch

import deterministic_invariant_gemm_amd as dig
import oracle
import synth
from parity import dev, host

pytestmark = pytest.mark.gpu

M, K, N = 524288, 4608, 64
SEED = 91
ROWS = np.array([0, 1, 262147, 466034, 500001, M - 2, M - 1], dtype=np.int64)
COLS = np.array([0, 1, 2305, K - 1], dtype=np.int64)


def bf16_bits(v: np.ndarray) -> np.ndarray:
    return synth.to_bits(v, synth.BF16)


@pytest.fixture(scope="module")
def big():
    assert 466034 * K * 2 > 2 ** 32  # sampled rows past 4 GiB of X
    print(f"large operands: generating X [{M}, {K}] on the GPU", flush=True)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    cols = torch.arange(K, device="cuda")
    for r0 in range(0, M, 32768):
        rows = torch.arange(r0, r0 + 32768, device="cuda")
        x[r0:r0 + 32768] = synth.hashed_ints(rows, cols, -4, 3, SEED, 0, xp=torch,
                                             device="cuda").to(torch.bfloat16)
    w = bf16_bits(synth.hashed_ints(np.arange(K), np.arange(N), -4, 3, SEED, 1))
    dy = bf16_bits(synth.hashed_ints(np.arange(M), np.arange(N), -1, 1, SEED, 2))
    torch.cuda.synchronize()
    return {"x": x.view(torch.int16), "w": w, "dy": dy, "w_d": dev(w), "dy_d": dev(dy)}


def x_rows(rows):
    return bf16_bits(synth.hashed_ints(rows, np.arange(K), -4, 3, SEED, 0))


def test_forward_beyond_4gib(big):
    print("large operands: forward", flush=True)
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    dig.check(dig.bi_forward(y, big["x"], big["w_d"], None, M, K, N, dig.BI_BF16,
                             torch.cuda.current_stream(), 1), "bi_forward")
    got = host(y[torch.from_numpy(ROWS).cuda()], np.uint16)
    res = oracle.linear_forward(synth.BF16, x_rows(ROWS), big["w"], None, len(ROWS), K, N)
    assert np.array_equal(got, res.out)
    # the generator agrees with itself across backends on these rows
    assert np.array_equal(host(big["x"][torch.from_numpy(ROWS).cuda()], np.uint16), x_rows(ROWS))


def test_dx_output_beyond_4gib(big):
    print("large operands: dX (4.8 GB output)", flush=True)
    dx = torch.empty((M, K), dtype=torch.int16, device="cuda")
    dig.check(dig.bi_backward_dx(dx, big["dy_d"], big["w_d"], M, K, N, dig.BI_BF16,
                                 torch.cuda.current_stream(), 1), "bi_backward_dx")
    got = host(dx[torch.from_numpy(ROWS).cuda()], np.uint16)
    del dx
    res = oracle.linear_dx(synth.BF16, big["dy"][ROWS], big["w"], len(ROWS), K, N)
    assert np.array_equal(got, res.out)


def test_dw_and_bias_grad_over_half_a_million_rows(big):
    print("large operands: dW (chunked) and bias gradient", flush=True)
    s = torch.cuda.current_stream()
    nb = dig.bi_backward_dw_workspace_bytes(M, K, N, dig.BI_BF16, 1)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dw = torch.empty((K, N), dtype=torch.int16, device="cuda")
    dig.check(dig.bi_backward_dw(dw, big["x"], big["dy_d"], M, K, N, dig.BI_BF16, ws, nb, s, 1),
              "bi_backward_dw")
    got = host(dw[torch.from_numpy(COLS).cuda()], np.uint16)
    xc = bf16_bits(synth.hashed_ints(np.arange(M), COLS, -4, 3, SEED, 0))
    res = oracle.linear_dw(synth.BF16, xc, big["dy"], M, len(COLS), N)
    assert np.array_equal(got, res.out)

    nb = dig.bi_bias_grad_workspace_bytes(M, N, dig.BI_BF16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    db = torch.empty(N, dtype=torch.int16, device="cuda")
    dig.check(dig.bi_bias_grad(db, big["dy_d"], M, N, dig.BI_BF16, ws, nb, s), "bi_bias_grad")
    assert np.array_equal(host(db, np.uint16), oracle.bias_grad(synth.BF16, big["dy"], M, N).out)


def e4m3_codes(v: np.ndarray) -> np.ndarray:
    """Small integers as e4m3fn codes (exact)."""
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_operand_beyond_4gib():
    m8, k8, n8 = 1048576, 4608, 64
    rows = np.array([0, 5, 524289, 1000003, m8 - 1], dtype=np.int64)
    assert 1000003 * k8 > 2 ** 32
    print(f"large operands: fp8 A [{m8}, {k8}] generated on the GPU", flush=True)
    a = torch.empty((m8, k8), dtype=torch.uint8, device="cuda")
    cols = torch.arange(k8, device="cuda")
    for r0 in range(0, m8, 32768):
        r = torch.arange(r0, r0 + 32768, device="cuda")
        a[r0:r0 + 32768] = synth.hashed_ints(r, cols, -8, 8, SEED, 3, xp=torch, device="cuda").to(
            torch.float8_e4m3fn).view(torch.uint8)
    bt = e4m3_codes(synth.hashed_ints(np.arange(n8), np.arange(k8), -8, 8, SEED, 4))
    da = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    db = torch.tensor([0.25], dtype=torch.float32, device="cuda")
    y = torch.empty((m8, n8), dtype=torch.int16, device="cuda")
    print("large operands: fp8 GEMM", flush=True)
    dig.check(dig.bi_fp8_mm(y, a, dev(bt), da, db, m8, k8, n8, torch.cuda.current_stream(), 1),
              "bi_fp8_mm")
    got = host(y[torch.from_numpy(rows).cuda()], np.uint16)
    a_rows = e4m3_codes(synth.hashed_ints(rows, np.arange(k8), -8, 8, SEED, 3))
    assert np.array_equal(host(a[torch.from_numpy(rows).cuda()], np.uint8), a_rows)
    res = oracle.fp8_mm(a_rows, bt, 0.5, 0.25, len(rows), k8, n8)
    assert np.array_equal(got, res.out)


def test_grouped_input_beyond_4gib(big):
    """The bf16 X above as the grouped GEMM's input (4 experts, padding rows
    at the end): segment-anchored register-staged tiles past 4 GiB."""
    print("large operands: grouped forward", flush=True)
    e = 4
    ids, offsets = synth.route(M, e, SEED, pad_rows=1000, idx=5)
    wts = bf16_bits(synth.hashed_ints(np.arange(e * N), np.arange(K), -4, 3, SEED, 6))
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    dig.check(dig.bi_grouped_nt(y, big["x"], dev(wts), dev(ids), dev(offsets), M, K, N, e,
                                dig.BI_BF16, torch.cuda.current_stream(), 1), "bi_grouped_nt")
    rows = np.concatenate([ROWS, [M - 1001, M - 1000]])  # the last routed row, the first padding row
    got = host(y[torch.from_numpy(rows).cuda()], np.uint16)
    res = oracle.grouped_fwd(synth.BF16, x_rows(rows), wts, ids[rows], len(rows), K, N, e)
    assert np.array_equal(got, res.out)
    assert not got[-1].any()  # padding row: exact +0


def test_f32_scalar_tier_beyond_4gib():
    """f32 always runs the scalar FMA tier: X f32 [524288, 2304] (4.8 GB)."""
    m, k, n = M, 2304, 64
    print(f"large operands: f32 X [{m}, {k}] on the scalar tier", flush=True)
    x = torch.empty((m, k), dtype=torch.float32, device="cuda")
    cols = torch.arange(k, device="cuda")
    for r0 in range(0, m, 32768):
        r = torch.arange(r0, r0 + 32768, device="cuda")
        x[r0:r0 + 32768] = synth.hashed_ints(r, cols, -4, 3, SEED, 7, xp=torch, device="cuda")
    w = synth.hashed_ints(np.arange(k), np.arange(n), -4, 3, SEED, 8).view(np.uint32)
    y = torch.empty((m, n), dtype=torch.int32, device="cuda")
    assert dig.bi_plan(dig.OP_FWD, dig.BI_F32, 1, k, n)[0] == 0
    dig.check(dig.bi_forward(y, x, dev(w), None, m, k, n, dig.BI_F32,
                             torch.cuda.current_stream(), 1), "bi_forward f32")
    got = host(y[torch.from_numpy(ROWS).cuda()], np.uint32)
    xr = synth.hashed_ints(ROWS, np.arange(k), -4, 3, SEED, 7).view(np.uint32)
    res = oracle.linear_forward(synth.F32, xr, w, None, len(ROWS), k, n)
    assert np.array_equal(got, res.out)
