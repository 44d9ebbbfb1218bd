"""Host-side checks of the C ABI: the library loads, exports every function
include/bi.h declares, and rejects invalid arguments before any HIP call.
No kernel is launched here (every call below returns during validation or is
an empty-batch no-op), so these run without a GPU."""
import ctypes
import os
import re

import pytest

import deterministic_invariant_gemm_amd as dig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "bi.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bi_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dig.LIB_PATH):
        from deterministic_invariant_gemm_amd import build
        build.build()
    return dig.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in list(range(-7, 1)):
        s = dig.status_string(code)
        assert s.startswith(dig.STATUS[code])
    assert "unknown" in dig.status_string(-99)


F = 12345 * 4096  # a non-null fake device address; never dereferenced


def test_validation_errors(lib):
    assert dig.bi_forward(F, F, F, None, 4, 4, 4, 7) == -2
    assert dig.bi_forward(F, F, F, None, -1, 4, 4, dig.BI_BF16) == -3
    assert dig.bi_forward(None, F, F, None, 4, 4, 4, dig.BI_BF16) == -1
    assert dig.bi_forward(F, None, F, None, 4, 4, 4, dig.BI_BF16) == -1
    assert dig.bi_forward(F, F, F, None, 1 << 30, 1 << 20, 4, dig.BI_BF16) == -4
    assert dig.bi_backward_dx(F, None, F, 4, 4, 4, dig.BI_F16) == -1
    assert dig.bi_backward_dx(F, F, F, 4, -4, 4, dig.BI_F16) == -3
    assert dig.bi_fp8_mm(F, F, F, None, F, 4, 4, 4) == -1
    assert dig.bi_fp8_mm(F, F, F, F, F, 4, -1, 4) == -3
    # grouped: k, n, e must be positive; offsets needed on the MFMA tier
    assert dig.bi_grouped_nt(F, F, F, F, F, 4, 0, 4, 2, dig.BI_BF16) == -3
    assert dig.bi_grouped_nt(F, F, F, F, F, 4, 4, 4, 0, dig.BI_BF16) == -3
    assert dig.bi_grouped_nt(F, F, F, F, None, 4, 128, 128, 2, dig.BI_BF16, tc=1) == -1
    assert dig.bi_grouped_nt(F, F, F, None, F, 4, 128, 128, 2, dig.BI_BF16) == -1
    assert dig.bi_grouped_nt_backward(F, F, F, F, F, F, None, 4, 8, 8, 2, dig.BI_BF16) == -1
    assert dig.bi_grouped_nt_backward(F, None, F, F, F, F, F, 4, 8, 8, 2, dig.BI_BF16) == -1


def test_dw_workspace_rules(lib):
    # small output (few tiles): the reduction over m is chunked, workspace needed
    m, k, n = 4096, 768, 48
    need = dig.bi_backward_dw_workspace_bytes(m, k, n, dig.BI_BF16, 1)
    tile, chunk = dig.bi_plan(dig.OP_DW, dig.BI_BF16, 1, k, n)
    assert tile == 0 and chunk > 0
    assert need == -(-m // chunk) * k * n * 4
    assert dig.bi_backward_dw(F, F, F, m, k, n, dig.BI_BF16, None, 0) == -5
    assert dig.bi_backward_dw(F, F, F, m, k, n, dig.BI_BF16, F, need - 1) == -5
    # one chunk: no workspace
    assert dig.bi_backward_dw_workspace_bytes(64, 128, 256, dig.BI_F32, 0) == 0
    # invalid arguments report 0 bytes
    assert dig.bi_backward_dw_workspace_bytes(-1, 4, 4, dig.BI_BF16, 1) == 0


def test_empty_batch_is_a_noop(lib):
    # m == 0: nothing to compute, nothing enqueued, success even with NULL data
    assert dig.bi_forward(None, None, None, None, 0, 16, 16, dig.BI_BF16) == 0
    assert dig.bi_backward_dx(None, None, None, 0, 16, 16, dig.BI_BF16) == 0
    assert dig.bi_fp8_mm(None, None, None, None, None, 0, 16, 16) == 0
    assert dig.bi_grouped_nt(None, None, None, None, None, 0, 16, 16, 2, dig.BI_BF16) == 0


def test_plan_is_shape_only_and_follows_fallback_rule(lib):
    # below 64 in a non-M output dim -> scalar tier; f32 -> scalar; tc=0 -> scalar
    assert dig.bi_plan(dig.OP_FWD, dig.BI_BF16, 1, 768, 48)[0] == 0
    assert dig.bi_plan(dig.OP_FWD, dig.BI_BF16, 1, 768, 3072)[0] > 0
    assert dig.bi_plan(dig.OP_FWD, dig.BI_F32, 1, 768, 3072)[0] == 0
    assert dig.bi_plan(dig.OP_FWD, dig.BI_BF16, 0, 768, 3072)[0] == 0
    assert dig.bi_plan(dig.OP_DX, dig.BI_BF16, 1, 768, 48)[0] > 0   # dX output dim is K
    assert dig.bi_plan(dig.OP_DX, dig.BI_BF16, 1, 48, 768)[0] == 0
    assert dig.bi_plan(dig.OP_DW, dig.BI_BF16, 1, 768, 48)[0] == 0
    assert dig.bi_plan(dig.OP_FP8, 0, 1, 4096, 4096)[0] > 0
    # the scalar-tier dW chunk does not depend on dtype (bf16 == upcast f32)
    for k, n in [(768, 48), (64, 64), (4096, 4096)]:
        assert dig.bi_plan(dig.OP_DW, dig.BI_BF16, 0, k, n) == dig.bi_plan(dig.OP_DW, dig.BI_F32, 0, k, n)


def test_plan_batch_follows_the_launch_model(lib):
    """The batch-dependent tile (bits never change with it): the default
    workload's forward on 256x192 and dX on 128x96, the 8192x4096x4096 forward
    on 256x256, the deep-stage narrow tiles for tiny batches, and the choices
    the launch model makes where forced-tile timings on MI355X found another
    tile fastest (forward 16384x2048x1408 on 256x192 (93 against 110 us for
    128x128), 4096x2048x1024 on 128x128 (20 against 27 us), dX with K = 1280
    on 256x96 (27 against 38 us))."""
    bf, fwd, dx, fp8 = dig.BI_BF16, dig.OP_FWD, dig.OP_DX, dig.OP_FP8
    assert dig.bi_plan_batch(fwd, bf, 1, 4096, 768, 3072) == 111
    assert dig.bi_plan_batch(dx, bf, 1, 4096, 768, 3072) == 45
    assert dig.bi_plan_batch(fwd, bf, 1, 8192, 4096, 4096) == 52
    assert dig.bi_plan_batch(fwd, bf, 1, 1, 4096, 4096) == 321
    assert dig.bi_plan_batch(fwd, bf, 1, 128, 4096, 4096) == 220
    assert dig.bi_plan_batch(dx, bf, 1, 17, 4096, 4096) == 120
    assert dig.bi_plan_batch(fwd, bf, 1, 16384, 2048, 1408) == 111
    assert dig.bi_plan_batch(fwd, bf, 1, 4096, 2048, 1024) == 44
    assert dig.bi_plan_batch(dx, bf, 1, 4096, 1280, 2048) == 50
    # outputs narrower than 128 columns keep the 64x64 tile at large batches
    assert dig.bi_plan_batch(fwd, bf, 1, 65536, 768, 96) == 46
    assert dig.bi_plan_batch(dig.OP_GFWD, bf, 1, 65536, 768, 96, 8) == 46
    # fp8 8192x4096x4096: 256x256 with eight waves (exact path; 201 against 204 us
    # for four waves of 128x128), the spread-copy 256x256 tile on the fp8
    # instruction (tc = 3); 4096x1024x4096 (K = 4096, N = 1024) on 128x128
    # (exact 32 against 40 us for the default)
    assert dig.bi_plan_batch(fp8, 0, 1, 8192, 4096, 4096) == 52
    assert dig.bi_plan_batch(fp8, 0, 3, 8192, 4096, 4096) == 112
    assert dig.bi_plan_batch(fp8, 0, 1, 4096, 4096, 1024) == 44
    assert dig.bi_plan_batch(fp8, 0, 1, 16, 4096, 4096) == 321
    assert dig.bi_plan_batch(fp8, 0, 3, 16, 4096, 4096) == 321
    # m == 0: the bi_plan tile; the scalar tier and bad arguments as in bi_plan
    assert dig.bi_plan_batch(fwd, bf, 1, 0, 768, 3072) == dig.bi_plan(fwd, bf, 1, 768, 3072)[0]
    assert dig.bi_plan_batch(fwd, bf, 1, 4096, 768, 48) == 0
    assert dig.bi_plan_batch(fwd, bf, 1, -1, 768, 3072) == -3
    assert dig.bi_plan_batch(fwd, 9, 1, 4096, 768, 3072) == dig.bi_plan(fwd, 9, 1, 768, 3072)[0]
    # grouped forward (e experts: one partial row tile per expert): 256x256 for
    # 32768 rows x 4096 columns (265 against 323 us for 256x192), 128x128 with
    # copy waves for 4096 x 4096 -> 2048 with 8 experts (73 against 143 us)
    gf = dig.OP_GFWD
    assert dig.bi_plan_batch(gf, bf, 1, 32768, 1024, 4096, 8) == 112
    assert dig.bi_plan_batch(gf, bf, 1, 4096, 4096, 2048, 8) == 44
    assert dig.bi_plan_batch(gf, bf, 1, 16384, 2048, 1408, -1) == -3
    # grouped dinput: 256x256 (sharing a launch with the 192x256 dweights tiles)
    # for 16384 rows of 2048 -> 1408, 128x128 with copy waves for 4096 rows of
    # 4096 -> 2048 with 8 experts (182 against 202 us for the backward)
    gd = dig.OP_GDIN
    assert dig.bi_plan_batch(gd, bf, 1, 16384, 2048, 1408, 8) == 52
    assert dig.bi_plan_batch(gd, bf, 1, 4096, 4096, 2048, 8) == 44
    # dW and the grouped dweights: the bi_plan tile at any batch
    for op in (dig.OP_DW, dig.OP_GDW):
        for m in (1, 4096, 65536):
            assert dig.bi_plan_batch(op, bf, 1, m, 2048, 1408, 8) == dig.bi_plan(op, bf, 1, 2048, 1408)[0]
    # every batch size of a sweep runs a tile that exists
    for m in (1, 2, 31, 64, 100, 256, 1000, 2049, 4096, 10000, 65536):
        for k, n in ((768, 3072), (4096, 4096), (1408, 2048), (2048, 1024)):
            assert dig.bi_plan_batch(fwd, bf, 1, m, k, n) in (44, 52, 53, 111, 120, 220, 321)
            assert dig.bi_plan_batch(dx, bf, 1, m, k, n) in (45, 50, 53, 55, 111, 120)
            assert dig.bi_plan_batch(fp8, 0, 1, m, k, n) in (44, 52, 54, 111, 120, 220, 321)
            assert dig.bi_plan_batch(fp8, 0, 3, m, k, n) in (41, 44, 111, 112, 115, 120, 220, 321)


def test_fp8_producer_validation(lib):
    assert dig.bi_fp8_quantize(F, F, F, None, 4, 7) == -2
    assert dig.bi_fp8_quantize(F, F, F, None, -1, dig.BI_FP8_E4M3) == -3
    assert dig.bi_fp8_quantize(None, F, F, None, 4, dig.BI_FP8_E5M2) == -1
    assert dig.bi_fp8_quantize(F, F, None, F, 4, dig.BI_FP8_E4M3) == -1
    assert dig.bi_fp8_quantize(None, None, None, None, 0, dig.BI_FP8_E4M3) == 0
    assert dig.bi_fp8_transpose_quantize(F, F, F, None, 4, -2, dig.BI_FP8_E4M3) == -3
    assert dig.bi_fp8_transpose_quantize(F, F, F, None, 65535 * 64 + 1, 1, 3) == -4
    assert dig.bi_fp8_transpose_quantize(F, F, F, None, 0, 9, dig.BI_FP8_E4M3) == 0
    # workspace: forward needs the two quantised operands, backward four plus
    # a scratch line; 256-byte aligned pieces
    a = lambda b: (b + 255) // 256 * 256
    m, k, n = 64, 32, 16
    fwd = a(m * k) + a(n * k)
    bwd = a(m * n) + a(k * n) + a(n * m) + a(k * m) + 256
    assert dig.bi_fp8_linear_workspace_bytes(m, k, n) == max(fwd, bwd)
    assert dig.bi_fp8_linear_workspace_bytes(-1, k, n) == 0
    ws = dig.bi_fp8_linear_workspace_bytes(m, k, n)
    assert dig.bi_fp8_linear_forward(F, F, F, None, F, F, F, None, None, None, m, k, n,
                                     F, ws) == -1
    assert dig.bi_fp8_linear_forward(F, F, F, None, F, F, F, F, None, None, m, k, n,
                                     F, 16) == -5
    assert dig.bi_fp8_linear_forward(F, F, F, None, F, F, F, F, None, None, m, -k, n,
                                     F, ws) == -3
    assert dig.bi_fp8_linear_backward(F, F, F, F, F, None, F, F, F, F, F, None, m, k, n,
                                      F, ws) == -1
    assert dig.bi_fp8_linear_backward(F, F, F, F, F, F, F, F, F, F, F, None, m, k, n,
                                      F, 100) == -5


def test_tc2_requires_the_mfma_tier(lib):
    """tc = 2 errors out where tc = 1 would fall back to the scalar tier;
    checked before any launch (the fake pointers are never touched)."""
    U = -7
    # f32 has no MFMA tier; narrow outputs fall back
    assert dig.bi_forward(F, F, F, None, 4, 128, 128, dig.BI_F32, None, 2) == U
    assert dig.bi_forward(F, F, F, None, 4, 128, 48, dig.BI_BF16, None, 2) == U
    assert dig.bi_backward_dx(F, F, F, 4, 48, 128, dig.BI_BF16, None, 2) == U
    assert dig.bi_backward_dw(F, F, F, 4, 128, 32, dig.BI_F16, None, 0, None, 2) == U
    assert dig.bi_fp8_mm(F, F, F, F, F, 4, 64, 32, None, 2) == U
    assert dig.bi_grouped_nt(F, F, F, F, F, 4, 128, 48, 2, dig.BI_BF16, None, 2) == U
    assert dig.bi_grouped_nt(F, F, F, F, F, 4, 128, 128, 2, dig.BI_F32, None, 2) == U
    assert dig.bi_grouped_nt_backward(F, F, F, F, F, F, F, 4, 40, 128, 2, dig.BI_BF16,
                                      None, 2) == U
    assert dig.bi_plan(0, dig.BI_BF16, 2, 768, 48)[0] == U
    assert dig.bi_plan(0, dig.BI_BF16, 2, 768, 64)[0] > 0
    # even an empty batch reports it (validation comes before the no-op)
    assert dig.bi_forward(F, F, F, None, 0, 128, 48, dig.BI_BF16, None, 2) == U
    assert dig.bi_backward_dw_workspace_bytes(9000, 128, 32, dig.BI_BF16, 2) == 0


def test_bias_grad_validation(lib):
    m, n = 1000, 300
    need = dig.bi_bias_grad_workspace_bytes(m, n, dig.BI_BF16)
    assert need == -(-m // 256) * n * 4
    assert dig.bi_bias_grad_workspace_bytes(256, n, dig.BI_BF16) == 0
    assert dig.bi_bias_grad_workspace_bytes(257, n, dig.BI_BF16) == 2 * n * 4
    assert dig.bi_bias_grad_workspace_bytes(-1, n, dig.BI_BF16) == 0
    assert dig.bi_bias_grad(F, F, m, n, dig.BI_BF16, None, 0) == -5
    assert dig.bi_bias_grad(F, F, m, n, dig.BI_BF16, F, need - 1) == -5
    assert dig.bi_bias_grad(F, F, m, n, dig.BI_BF16, F + 2, need) == -5  # misaligned
    assert dig.bi_bias_grad(F, F, m, n, 7, F, need) == -2
    assert dig.bi_bias_grad(F, F, -1, n, dig.BI_BF16, F, need) == -3
    assert dig.bi_bias_grad(None, F, m, n, dig.BI_BF16, F, need) == -1
    assert dig.bi_bias_grad(F, None, m, n, dig.BI_BF16, F, need) == -1
    assert dig.bi_bias_grad(F, F, 1 << 30, 1 << 20, dig.BI_BF16, F, need) == -4
    assert dig.bi_bias_grad(None, None, 5, 0, dig.BI_BF16, None, 0) == 0  # n == 0: no-op


def test_linear_backward_validation(lib):
    """bi_linear_backward checks every argument of both gradients before
    anything is enqueued."""
    bf = dig.BI_BF16
    assert dig.bi_linear_backward(None, None, F, F, F, 4, 8, 8, bf, None, 0) == -1
    assert dig.bi_linear_backward(F, F, F, F, F, 4, 8, 8, 9, None, 0) == -2
    assert dig.bi_linear_backward(F, F, F, F, F, 4, -8, 8, bf, None, 0) == -3
    assert dig.bi_linear_backward(F, F, None, F, F, 4, 128, 128, bf, None, 0) == -1
    assert dig.bi_linear_backward(F, F, F, None, F, 4, 128, 128, bf, None, 0) == -1
    assert dig.bi_linear_backward(F, F, F, F, F, 1 << 30, 1 << 20, 4, bf, None, 0) == -4
    # dW chunked (few output tiles): the workspace is checked before dX runs
    m, k, n = 4096, 768, 48
    need = dig.bi_backward_dw_workspace_bytes(m, k, n, bf, 1)
    assert need > 0
    assert dig.bi_linear_backward(F, F, F, F, F, m, k, n, bf, None, 0) == -5
    assert dig.bi_linear_backward(F, F, F, F, F, m, k, n, bf, F, need - 1) == -5
    # tc = 2 where dX (output dim k = 48) would fall back to the scalar tier
    assert dig.bi_plan(dig.OP_DX, bf, 1, 48, 768)[0] == 0
    assert dig.bi_linear_backward(F, F, F, F, F, 64, 48, 768, bf, None, 0, tc=2) == -7
    # nothing to compute; NULL outputs are fine when both are empty
    assert dig.bi_linear_backward(F, F, None, None, None, 0, 0, 16, bf, None, 0) == 0
    assert dig.bi_linear_backward(None, None, None, None, None, 64, 0, 128, bf, None, 0) == 0
    assert dig.bi_linear_backward(None, None, None, None, None, 0, 96, 0, bf, None, 0) == 0
    assert dig.bi_linear_backward(None, None, F, F, F, 0, 96, 128, bf, None, 0) == -1


def test_tc_values(lib):
    """tc: 0 scalar, 1 auto, 2 MFMA required, 3 fp8 GEMMs on the fp8 matrix
    instruction (other ops reject it); every other value is rejected by
    libbi.so, while libbi_testing.so takes tc = 16 + tile id (plus 4096 for the
    fp8 fast path) and reports the forced tile in the plan."""
    U, bf = -7, dig.BI_BF16
    for tc in (0, 1, 2):
        assert dig.bi_plan(dig.OP_FWD, bf, tc, 768, 3072)[0] >= 0
    exact = dig.bi_plan(dig.OP_FP8, bf, 1, 4096, 4096)[0]
    fast = dig.bi_plan(dig.OP_FP8, bf, dig.TC_FP8_FAST, 4096, 4096)[0]
    assert exact > 0 and fast > 0
    assert dig.bi_plan(dig.OP_FWD, bf, dig.TC_FP8_FAST, 768, 3072)[0] == U
    assert dig.bi_forward(F, F, F, None, 4, 128, 128, bf, None, dig.TC_FP8_FAST) == U
    assert dig.bi_backward_dx(F, F, F, 4, 128, 128, bf, None, 16 + 44) == U
    for tc in (4, 15, 16 + 44, 4096 + 16 + 44, -1):
        assert dig.bi_plan(dig.OP_FWD, bf, tc, 768, 3072)[0] == U, tc
        assert dig.bi_plan(dig.OP_FP8, bf, tc, 4096, 4096)[0] == U, tc
    # n < 64: tc = 3 falls back to the scalar tier like tc = 1
    assert dig.bi_plan(dig.OP_FP8, bf, dig.TC_FP8_FAST, 4096, 48)[0] == 0
    if not os.path.exists(dig.LIB_TESTING_PATH):
        pytest.skip("libbi_testing.so not built")
    with dig.testing_build():
        assert dig.bi_plan(dig.OP_FWD, bf, 16 + 44, 768, 3072)[0] == 44
        assert dig.bi_plan(dig.OP_FP8, bf, 16 + 112, 4096, 4096)[0] == 112
        assert dig.bi_plan(dig.OP_FP8, bf, 4096 + 16 + 54, 4096, 4096)[0] == 54
        # the fast bit is for fp8 GEMMs only; the dW chunk never follows a forced tile
        assert dig.bi_plan(dig.OP_FWD, bf, 4096 + 16 + 44, 768, 3072)[0] == U
        assert (dig.bi_plan(dig.OP_DW, bf, 16 + 46, 768, 3072)[1]
                == dig.bi_plan(dig.OP_DW, bf, 1, 768, 3072)[1])
    # back on the production library
    assert dig.bi_plan(dig.OP_FWD, bf, 16 + 44, 768, 3072)[0] == U


def test_static_backward_validation(lib):
    """bi_linear_backward_static refuses partials beyond its static array and
    reports bi_linear_backward's validation errors, all before any HIP call."""
    bf = dig.BI_BF16
    m, k, n = 65536, 1024, 1024  # 64 chunks of 1024 x 1024 f32 partials: 256 MiB
    assert dig.bi_backward_dw_workspace_bytes(m, k, n, bf, 1) > dig.BI_STATIC_SCRATCH_BYTES
    assert dig.bi_linear_backward_static(F, F, F, F, F, m, k, n, bf, None, 1) == -5
    assert dig.bi_linear_backward_static(F, F, F, F, F, 4, 8, 8, 9, None, 1) == -2
    assert dig.bi_linear_backward_static(F, F, F, F, F, 4, -8, 8, bf, None, 1) == -3
    assert dig.bi_linear_backward_static(F, F, None, F, F, 4, 128, 128, bf, None, 1) == -1
    assert dig.bi_linear_backward_static(F, F, F, F, F, 64, 48, 768, bf, None, 2) == -7
    assert dig.bi_linear_backward_static(None, None, None, None, None, 0, 96, 0, bf,
                                         None, 1) == 0
