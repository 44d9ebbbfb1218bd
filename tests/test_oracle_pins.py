"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties one part of the oracle to something it cannot agree with by
construction: the closed-form definitions of the number formats (checked
exhaustively against torch / numpy casts), exact rational rounding, hand-derived
cases, an independent numpy float64 matmul, finite differences of the loss, and
the structural properties the pages state (padding rows are zero, dweights are
f32, an empty expert has zero gradient).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


# ---------------------------------------------------------------------------
# codecs: exhaustive against library casts
# ---------------------------------------------------------------------------

def _same(a, b):
    return (np.isnan(a) and np.isnan(b)) or a == b


def test_decode_e4m3_exhaustive_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        assert _same(oracle.decode_e4m3(c), ref[c]), hex(c)
    # facts of the OCP e4m3fn format
    assert oracle.decode_e4m3(0x7E) == 448.0
    assert oracle.decode_e4m3(0x08) == 2.0 ** -6
    assert oracle.decode_e4m3(0x01) == 2.0 ** -9
    assert np.isnan(oracle.decode_e4m3(0x7F)) and np.isnan(oracle.decode_e4m3(0xFF))


def test_decode_f16_exhaustive_vs_numpy():
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    L = oracle.lib()
    for c in range(65536):
        assert _same(L.orc_decode_f16(c), ref[c]), hex(c)


def test_decode_bf16_exhaustive_vs_torch():
    # int32 -> int16 wraps, so element c holds the bit pattern c
    ref = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16) \
        .to(torch.float64).numpy()
    L = oracle.lib()
    for c in range(65536):
        assert _same(L.orc_decode_bf16(c), ref[c]), hex(c)


# ---------------------------------------------------------------------------
# RNE encoders: against exact rational rounding
# ---------------------------------------------------------------------------

def _exact_round(x: float, p: int, emin: int, max_finite: Fraction):
    """Correct rounding of x to a binary format, by exact rational arithmetic:
    find the two representable neighbours and pick the nearer one, ties to the
    one with an even last significand bit."""
    fx = Fraction(x)
    if fx == 0:
        return Fraction(0)
    sgn = -1 if fx < 0 else 1
    ax = abs(fx)
    e = ax.numerator.bit_length() - ax.denominator.bit_length()
    while Fraction(2) ** e > ax:
        e -= 1
    while Fraction(2) ** (e + 1) <= ax:
        e += 1
    q = Fraction(2) ** (max(e, emin) - (p - 1))
    lo = (ax / q).__floor__()
    rem = ax / q - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * q
    if r > max_finite:
        return sgn * Fraction(10) ** 400  # stands for infinity
    return sgn * r


def _decoded_or_inf(v):
    if np.isinf(v):
        return (1 if v > 0 else -1) * Fraction(10) ** 400
    return Fraction(v)


def _random_doubles(n, lo_exp, hi_exp, seed):
    g = np.random.default_rng(seed)
    mant = g.uniform(1.0, 2.0, size=n)
    ex = g.integers(lo_exp, hi_exp + 1, size=n)
    sign = g.choice([-1.0, 1.0], size=n)
    return sign * np.ldexp(mant, ex)


BF16_MAX = Fraction(255, 128) * Fraction(2) ** 127
F16_MAX = Fraction(65504)


@pytest.mark.parametrize("seed", [0, 1])
def test_rne_bf16_vs_exact_rational(seed):
    xs = list(_random_doubles(4000, -140, 130, seed))
    # exact ties and near-ties around representable values
    for base in (1.0, 3.0, 2.0 ** -126, 2.0 ** -133 * 5, 2.0 ** 127 * 1.9921875):
        ulp = 2.0 ** (max(math.frexp(base)[1] - 1, -126) - 7)
        for d in (0.5, 0.5 + 2 ** -20, 0.5 - 2 ** -20, 1.5, 0.25):
            xs += [base + d * ulp, -(base + d * ulp)]
    for x in map(float, xs):
        got = _decoded_or_inf(oracle.decode_bf16(oracle.rne_bf16(x)))
        assert got == _exact_round(x, 8, -126, BF16_MAX), x


@pytest.mark.parametrize("seed", [0, 1])
def test_rne_f16_vs_exact_rational_and_numpy(seed):
    xs = list(_random_doubles(4000, -27, 17, seed))
    xs += [65504.0, 65519.99, 65520.0, 65535.0, 2.0 ** -24 * 1.5, 2.0 ** -25,
           2.0 ** -25 * 1.0000001, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11]
    for x in map(float, xs):
        bits = oracle.rne_f16(x)
        got = _decoded_or_inf(oracle.decode_f16(bits))
        assert got == _exact_round(x, 11, -14, F16_MAX), x
        # numpy's double -> half conversion is an independent correctly
        # rounded implementation
        assert bits == int(np.array([x]).astype(np.float16).view(np.uint16)[0]), x


def test_rne_f32_vs_exact_rational():
    xs = list(_random_doubles(4000, -155, 130, 7))
    xs += [1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 1 + 2.0 ** -24 + 2.0 ** -40]
    fmax = Fraction(2 ** 24 - 1, 2 ** 23) * Fraction(2) ** 127
    for x in map(float, xs):
        got = _decoded_or_inf(oracle.lib().orc_decode_f32_bits(oracle.rne_f32(x)))
        assert got == _exact_round(x, 24, -126, fmax), x


def test_rne_hand_ties():
    # values from the definition of round-to-nearest-even
    assert oracle.rne_bf16(1 + 2.0 ** -8) == 0x3F80
    assert oracle.rne_bf16(1 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.rne_bf16(-(1 + 2.0 ** -8)) == 0xBF80
    assert oracle.rne_bf16(2.0 ** 128) == 0x7F80
    assert oracle.rne_f16(1 + 2.0 ** -11) == 0x3C00
    assert oracle.rne_f16(65520.0) == 0x7C00
    assert oracle.rne_f16(65519.0) == 0x7BFF
    assert oracle.rne_e4m3_sat(1 + 2.0 ** -4) == 0x38
    assert oracle.rne_e4m3_sat(1e9) == 0x7E
    assert oracle.rne_bf16(-0.0) == 0x8000 and oracle.rne_bf16(0.0) == 0


def test_rne_does_not_round_through_f32():
    # 1 + 2^-8 + 2^-30: through f32 it would become 1 + 2^-8 (a tie) and then
    # 1.0; rounded once it is above the midpoint and goes to 1 + 2^-7.
    assert oracle.rne_bf16(1 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81


# ---------------------------------------------------------------------------
# hand-derived GEMMs
# ---------------------------------------------------------------------------

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["linear"], ids=lambda c: c["name"])
def test_golden_linear(case):
    dt, m, k, n = case["dt"], case["m"], case["k"], case["n"]
    st = oracle.STORAGE[dt]
    x = np.array(case["x"], dtype=st).reshape(m, k)
    w = np.array(case["w"], dtype=st).reshape(k, n)
    b = None if case["b"] is None else np.array(case["b"], dtype=st)
    y = oracle.linear_forward(dt, x, w, b, m, k, n, threads=1).out
    assert y.ravel().tolist() == case["y"]
    if "dx" in case:
        dy = np.array(case["dy"], dtype=st).reshape(m, n)
        assert oracle.linear_dx(dt, dy, w, m, k, n).out.ravel().tolist() == case["dx"]
        assert oracle.linear_dw(dt, x, dy, m, k, n).out.ravel().tolist() == case["dw"]


@pytest.mark.parametrize("case", _golden()["fp8"], ids=lambda c: c["name"])
def test_golden_fp8(case):
    m, k, n = case["m"], case["k"], case["n"]
    a8 = np.array(case["a8"], dtype=np.uint8).reshape(m, k)
    bt8 = np.array(case["bt8"], dtype=np.uint8).reshape(n, k)
    y = oracle.fp8_mm(a8, bt8, case["da"], case["db"], m, k, n).out
    assert y.ravel().tolist() == case["y"]


@pytest.mark.parametrize("case", _golden()["grouped"], ids=lambda c: c["name"])
def test_golden_grouped(case):
    dt, m, k, n, e = case["dt"], case["m"], case["k"], case["n"], case["e"]
    inp = np.array(case["input"], dtype=np.uint16).reshape(m, k)
    wts = np.array(case["weights"], dtype=np.uint16)
    ids = np.array(case["row_experts"], dtype=np.uint32)
    dy = np.array(case["dy"], dtype=np.uint16).reshape(m, n)
    assert oracle.grouped_fwd(dt, inp, wts, ids, m, k, n, e).out.ravel().tolist() == case["y"]
    assert oracle.grouped_dinput(dt, dy, wts, ids, m, k, n, e).out.ravel().tolist() \
        == case["dinput"]
    assert oracle.grouped_dweights(dt, inp, dy, ids, m, k, n, e).out.ravel().tolist() \
        == case["dweights"]


# ---------------------------------------------------------------------------
# cross-checks against an independent float64 matmul (numpy / BLAS)
# ---------------------------------------------------------------------------

def _f64(bits, dt):
    return synth.to_f32(bits, dt).astype(np.float64)


def _check_vs_numpy(res, ref_s):
    # S: the same exact products summed in another order (BLAS blocking)
    # agree to a few f64 ulps of A
    assert np.all(np.abs(res.s - ref_s) <= 1e-13 * res.a + 1e-300)


@pytest.mark.parametrize("dt", [synth.F32, synth.BF16, synth.F16])
def test_linear_vs_numpy_float64(dt):
    d = synth.linear(37, 53, 29, dt, seed=11)
    m, k, n = d["m"], d["k"], d["n"]
    X, W, B, DY = (_f64(d[t], dt) for t in ("x", "w", "b", "dy"))
    f = oracle.linear_forward(dt, d["x"], d["w"], d["b"], m, k, n)
    _check_vs_numpy(f, X @ W + B)
    gx = oracle.linear_dx(dt, d["dy"], d["w"], m, k, n)
    _check_vs_numpy(gx, DY @ W.T)
    gw = oracle.linear_dw(dt, d["x"], d["dy"], m, k, n)
    _check_vs_numpy(gw, X.T @ DY)
    # A is the sum of |products| (+|bias|)
    assert np.allclose(f.a, np.abs(X) @ np.abs(W) + np.abs(B), rtol=1e-13)
    assert np.allclose(gx.a, np.abs(DY) @ np.abs(W).T, rtol=1e-13)
    assert np.allclose(gw.a, np.abs(X).T @ np.abs(DY), rtol=1e-13)


def test_rounded_outputs_vs_torch_cast_of_numpy_value():
    # The output bits are RNE(S).  Away from ties the f64 numpy value rounds
    # to the same bits through torch's f64 -> f32 -> bf16 path unless the
    # double rounding hits; count agreement over many elements.
    dt = synth.BF16
    d = synth.linear(64, 96, 80, dt, seed=12, bias=False)
    m, k, n = d["m"], d["k"], d["n"]
    X, W = _f64(d["x"], dt), _f64(d["w"], dt)
    res = oracle.linear_forward(dt, d["x"], d["w"], None, m, k, n)
    ref = torch.from_numpy(X @ W).to(torch.float32).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)
    assert np.mean(res.out == ref) > 0.999


def test_fp8_vs_numpy_float64():
    d = synth.fp8(23, 70, 19, seed=13)
    A = torch.from_numpy(d["a8"]).view(torch.float8_e4m3fn).double().numpy()
    B = torch.from_numpy(d["bt8"]).view(torch.float8_e4m3fn).double().numpy()
    r = oracle.fp8_mm(d["a8"], d["bt8"], d["da"], d["db"], d["m"], d["k"], d["n"])
    ref = (A @ B.T) * float(d["da"]) * float(d["db"])
    assert np.all(np.abs(r.s - ref) <= 1e-13 * r.a)


# ---------------------------------------------------------------------------
# finite differences of the loss  L = sum dY * (X W + b)
# ---------------------------------------------------------------------------

def test_dx_dw_are_finite_differences_of_forward():
    """L is linear in each element of X and W, so a central difference with
    a dyadic step on small-integer f32 operands is exact and must equal the
    oracle's dX and dW entries (index conventions and transposes included)."""
    dt = synth.F32
    m, k, n = 5, 4, 3
    d = synth.linear_integer(m, k, n, dt, seed=14)
    dy = _f64(d["dy"], dt)

    def loss(xb, wb):
        s = oracle.linear_forward(dt, xb, wb, d["b"], m, k, n).s
        return float(np.sum(dy * s))

    gx = oracle.linear_dx(dt, d["dy"], d["w"], m, k, n).s
    gw = oracle.linear_dw(dt, d["x"], d["dy"], m, k, n).s
    X, W = _f64(d["x"], dt), _f64(d["w"], dt)
    h = 0.5
    for i in range(m):
        for j in range(k):
            xp, xm = X.copy(), X.copy()
            xp[i, j] += h
            xm[i, j] -= h
            fd = (loss(synth.to_bits(xp.astype(np.float32), dt), d["w"])
                  - loss(synth.to_bits(xm.astype(np.float32), dt), d["w"])) / (2 * h)
            assert fd == gx[i, j]
    for i in range(k):
        for j in range(n):
            wp, wm = W.copy(), W.copy()
            wp[i, j] += h
            wm[i, j] -= h
            fd = (loss(d["x"], synth.to_bits(wp.astype(np.float32), dt))
                  - loss(d["x"], synth.to_bits(wm.astype(np.float32), dt))) / (2 * h)
            assert fd == gw[i, j]


def test_grouped_grads_are_finite_differences():
    dt = synth.F32
    m, k, n, e = 6, 3, 2, 3
    ids = np.array([0, 0, 1, 2, 2, synth.PAD_ID], dtype=np.uint32)
    inp = synth.integer_bits((m, k), -3, 3, 15, 0, dt)
    wts = synth.integer_bits((e, n, k), -3, 3, 15, 1, dt)
    dyb = synth.integer_bits((m, n), -3, 3, 15, 2, dt)
    dy = _f64(dyb, dt)

    def loss(ib, wb):
        return float(np.sum(dy * oracle.grouped_fwd(dt, ib, wb, ids, m, k, n, e).s))

    gi = oracle.grouped_dinput(dt, dyb, wts, ids, m, k, n, e).s
    gw = oracle.grouped_dweights(dt, inp, dyb, ids, m, k, n, e).s.reshape(e, n, k)
    I, Wt = _f64(inp, dt), _f64(wts, dt)
    for idx in np.ndindex(m, k):
        p, q = I.copy(), I.copy()
        p[idx] += 1
        q[idx] -= 1
        fd = (loss(synth.to_bits(p.astype(np.float32), dt), wts)
              - loss(synth.to_bits(q.astype(np.float32), dt), wts)) / 2
        assert fd == gi[idx]
    for idx in np.ndindex(e, n, k):
        p, q = Wt.copy(), Wt.copy()
        p[idx] += 1
        q[idx] -= 1
        fd = (loss(inp, synth.to_bits(p.astype(np.float32), dt))
              - loss(inp, synth.to_bits(q.astype(np.float32), dt))) / 2
        assert fd == gw[idx]


# ---------------------------------------------------------------------------
# the stated equivalence and structural properties
# ---------------------------------------------------------------------------

def test_bf16_equals_upcast_f32_then_rne_except_double_rounding():
    """Scalar-tier statement: bf16 == upcast -> f32 -> RNE downcast.  For the
    exact-sum oracle this holds except where the f32 value of S lands exactly
    on a bf16 midpoint (double rounding); such elements must differ by one
    ulp and must be rare."""
    d = synth.linear(48, 512, 64, synth.BF16, seed=16, sigma_w=0.02)
    m, k, n = d["m"], d["k"], d["n"]
    yb = oracle.linear_forward(synth.BF16, d["x"], d["w"], d["b"], m, k, n)
    up = {t: synth.to_bits(synth.to_f32(d[t], synth.BF16), synth.F32) for t in ("x", "w", "b")}
    yf = oracle.linear_forward(synth.F32, up["x"], up["w"], up["b"], m, k, n)
    assert np.array_equal(yf.s, yb.s)
    via = synth.to_bits(synth.to_f32(yf.out, synth.F32), synth.BF16)
    diff = np.nonzero(via != yb.out)
    assert len(diff[0]) <= 3
    for i, j in zip(*diff):
        assert abs(int(via[i, j]) - int(yb.out[i, j])) == 1


def test_grouped_padding_rows_are_zero_bytes_and_empty_expert_zero():
    d = synth.grouped(200, 40, 24, 5, synth.BF16, seed=17, pad_rows=23, empty=(2,))
    m, k, n, e = d["m"], d["k"], d["n"], d["e"]
    ids = d["row_experts"]
    y = oracle.grouped_fwd(synth.BF16, d["input"], d["weights"], ids, m, k, n, e).out
    di = oracle.grouped_dinput(synth.BF16, d["dy"], d["weights"], ids, m, k, n, e).out
    dw = oracle.grouped_dweights(synth.BF16, d["input"], d["dy"], ids, m, k, n, e).out \
        .reshape(e, n, k)
    pad = ids >= e
    assert pad.sum() == 23
    assert np.all(y[pad] == 0) and np.all(di[pad] == 0)
    assert np.all(dw[2] == 0)
    assert not np.all(dw[1] == 0)


def test_grouped_single_expert_reduces_to_linear():
    """E = 1 without padding: the grouped forward is X W with W = Wt[0]^T,
    and dinput is dY Wt[0] = dX of that linear; bit-equal."""
    dt = synth.BF16
    m, k, n = 33, 21, 17
    d = synth.grouped(m, k, n, 1, dt, seed=18)
    w_lin = np.ascontiguousarray(d["weights"][0].T)  # [k, n] = [in, out]
    y_g = oracle.grouped_fwd(dt, d["input"], d["weights"], d["row_experts"], m, k, n, 1).out
    y_l = oracle.linear_forward(dt, d["input"], w_lin, None, m, k, n).out
    assert np.array_equal(y_g, y_l)
    dx_g = oracle.grouped_dinput(dt, d["dy"], d["weights"], d["row_experts"], m, k, n, 1).out
    dx_l = oracle.linear_dx(dt, d["dy"], w_lin, m, k, n).out
    assert np.array_equal(dx_g, dx_l)
    dw_g = oracle.grouped_dweights(dt, d["input"], d["dy"], d["row_experts"], m, k, n, 1)
    dw_l = oracle.linear_dw(dt, d["input"], d["dy"], m, k, n)  # [k, n]
    assert np.array_equal(dw_g.s, dw_l.s.T)


def test_grouped_dweights_vs_numpy_per_expert():
    dt = synth.BF16
    d = synth.grouped(150, 30, 20, 4, dt, seed=19, pad_rows=9)
    m, k, n, e = d["m"], d["k"], d["n"], d["e"]
    ids = d["row_experts"]
    I, G = _f64(d["input"], dt), _f64(d["dy"], dt)
    r = oracle.grouped_dweights(dt, d["input"], d["dy"], ids, m, k, n, e)
    s = r.s.reshape(e, n, k)
    for j in range(e):
        sel = ids == j
        ref = G[sel].T @ I[sel]
        assert np.all(np.abs(s[j] - ref) <= 1e-13 * r.a.reshape(e, n, k)[j] + 1e-300)
    # output is f32 rounding of S
    assert np.array_equal(r.out, synth.to_bits(r.s.astype(np.float32), synth.F32))


def test_row_selection_matches_full_computation():
    d = synth.linear(40, 24, 16, synth.BF16, seed=20)
    m, k, n = d["m"], d["k"], d["n"]
    full = oracle.linear_forward(synth.BF16, d["x"], d["w"], d["b"], m, k, n, threads=3)
    rows = [39, 0, 7, 7, 21]
    part = oracle.linear_forward(synth.BF16, d["x"], d["w"], d["b"], m, k, n, rows=rows,
                                 threads=2)
    assert np.array_equal(part.out, full.out[rows])
    assert np.array_equal(part.s, full.s[rows])


def test_empty_reduction_is_positive_zero_plus_bias():
    # k = 0: Y = RNE(b); dW over m = 0 rows is +0
    dt = synth.BF16
    b = synth.normal_bits((5,), 1.0, 21, 0, dt)
    y = oracle.linear_forward(dt, np.zeros((3, 0), np.uint16), np.zeros((0, 5), np.uint16), b,
                              3, 0, 5)
    assert np.array_equal(y.out, np.tile(b, (3, 1)))
    dw = oracle.linear_dw(dt, np.zeros((0, 4), np.uint16), np.zeros((0, 5), np.uint16), 0, 4, 5)
    assert np.all(dw.out == 0)


# ---------------------------------------------------------------------------
# fp8 producer side: e5m2, quantisation, scaled fp8 linear
# ---------------------------------------------------------------------------

def test_decode_e5m2_exhaustive_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    for c in range(256):
        assert _same(oracle.decode_e5m2(c), ref[c]), hex(c)
    assert oracle.decode_e5m2(0x7B) == 57344.0          # largest finite
    assert oracle.decode_e5m2(0x7C) == math.inf
    assert oracle.decode_e5m2(0x01) == 2.0 ** -16       # smallest subnormal
    assert oracle.decode_e5m2(0x04) == 2.0 ** -14       # smallest normal


E4M3_MAX, E5M2_MAX = Fraction(448), Fraction(57344)


def _exact_round_sat(x, p, emin, max_finite):
    r = _exact_round(x, p, emin, max_finite)
    # _exact_round reports overflow as +-10^400; saturation keeps the sign
    return (max_finite if x > 0 else -max_finite) if abs(r) > max_finite else r


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_encoders_vs_exact_rational_and_torch(fmt):
    enc, dec = ((oracle.rne_e4m3_sat, oracle.decode_e4m3) if fmt == "e4m3"
                else (oracle.rne_e5m2_sat, oracle.decode_e5m2))
    p, emin, mx = (4, -6, E4M3_MAX) if fmt == "e4m3" else (3, -14, E5M2_MAX)
    tdt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    xs = list(_random_doubles(3000, emin - 4, 18, 11))
    # every representable value and every midpoint between neighbours
    vals = sorted({dec(c) for c in range(256) if math.isfinite(dec(c)) and dec(c) >= 0})
    xs += vals + [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    xs += [-v for v in xs] + [1e30, -1e30, float(mx) * 1.03, float(mx) * 1.1]
    for x in map(float, xs):
        code = enc(x)
        assert dec(code) == _exact_round_sat(x, p, emin, mx), (fmt, x)
        # torch's cast is an independent correctly rounded conversion (it
        # does not saturate, so only in-range values are compared)
        if abs(x) <= float(mx) and x != 0.0:
            ref = int(torch.tensor([x], dtype=torch.float64).to(tdt).view(torch.uint8)[0])
            assert code == ref, (fmt, x)


def _bf16(vals):
    return synth.to_bits(np.asarray(vals, dtype=np.float32), synth.BF16)


def test_quantize_hand_cases():
    # bf16 sources times scale_inv = 2, e4m3fn codes written out by hand from
    # the format definition: 2.0 = 0x40, -3.0 = 0xC4, 6.0 = 0x4C, +0, -0, 2000
    # saturates to 448 = 0x7E, 2^-9 is the smallest subnormal 0x01
    src = _bf16([1.0, -1.5, 3.0, 0.0, -0.0, 1000.0, 2.0 ** -10])
    codes, amax = oracle.fp8_quantize(oracle.E4M3, src, 2.0)
    assert list(codes) == [0x40, 0xC4, 0x4C, 0x00, 0x80, 0x7E, 0x01]
    assert amax == 1000.0
    # e5m2: 2.0 = 0x40, -3.0 = 0xC2, 6.0 = 0x46, 2000 = 1.953125 * 2^10 ->
    # RNE to 2048 = 0x68 (1.75*2^10 = 1792 and 2048 are the neighbours)
    codes, _ = oracle.fp8_quantize(oracle.E5M2, src, 2.0)
    assert list(codes[[0, 1, 2, 5]]) == [0x40, 0xC2, 0x46, 0x68]
    # transposed: [2,3] -> [3,2], element (r, c) lands at (c, r)
    src = _bf16([[1.0, 2.0, 4.0], [-1.0, -2.0, 0.5]])
    t, amax = oracle.fp8_transpose_quantize(oracle.E4M3, src, 1.0, 2, 3)
    assert t.tolist() == [[0x38, 0xB8], [0x40, 0xC0], [0x48, 0x30]] and amax == 4.0


def test_quantize_rounds_the_product_to_f32_first():
    # raw = 1 + 2^-7 (bf16), scale_inv = the f32 value just above
    # 1.0625 / raw.  The exact product is a hair above the e4m3 midpoint
    # 1.0625 (between 1.0 and 1.125) and would round up; rounded to f32 first
    # it is exactly the midpoint and goes to the even neighbour 1.0 (0x38).
    raw = Fraction(1) + Fraction(1, 128)
    target = Fraction(17, 16) / raw
    s = np.float32(float(target))
    if Fraction(float(s)) < target:
        s = np.nextafter(s, np.float32(2))
    prod = raw * Fraction(float(s))
    assert prod > Fraction(17, 16) and prod - Fraction(17, 16) < Fraction(1, 2 ** 24)
    codes, _ = oracle.fp8_quantize(oracle.E4M3, _bf16([1 + 2.0 ** -7]), float(s))
    assert codes[0] == 0x38


def _torch_quant(bits, scale_inv, dt=torch.float8_e4m3fn):
    """Independent quantisation: f32 product by torch, then torch's fp8 cast
    (values stay inside the format's range here, where it agrees with the
    saturating rule)."""
    f = torch.from_numpy(synth.to_f32(bits, synth.BF16).astype(np.float32))
    q = (f * torch.tensor(np.float32(scale_inv))).to(dt)
    return q.to(torch.float64).numpy()


def test_fp8_linear_forward_vs_numpy():
    m, k, n = 37, 150, 29
    d = synth.linear(m, k, n, synth.BF16, seed=5, sigma_w=1.0)
    x, b = d["x"], d["b"]
    w = synth.normal_bits((n, k), 1.0, 5, 9, synth.BF16)        # [N,K]
    sx_inv, sw_inv, sx, sw = 96.0, 80.0, 1 / 96.0, 1 / 80.0
    r = oracle.fp8_linear_forward(x, w, b, sx, sw, sx_inv, sw_inv, m, k, n)
    qx, qw = _torch_quant(x, sx_inv), _torch_quant(w, sw_inv)
    S = (qx @ qw.T) * float(np.float32(sx)) * float(np.float32(sw)) \
        + synth.to_f32(b, synth.BF16).astype(np.float64)
    assert np.allclose(r.s, S, rtol=1e-12, atol=1e-12)
    assert r.amax_x == np.abs(synth.to_f32(x, synth.BF16)).max()
    assert r.amax_w == np.abs(synth.to_f32(w, synth.BF16)).max()
    # integer codes with unit scales: every step exact, so the rounded output
    # is the exact integer result
    xi = _bf16(np.random.default_rng(3).integers(-6, 7, (m, k)))
    wi = _bf16(np.random.default_rng(4).integers(-6, 7, (n, k)))
    bi = _bf16(np.random.default_rng(5).integers(-9, 10, n))
    r = oracle.fp8_linear_forward(xi, wi, bi, 1.0, 1.0, 1.0, 1.0, m, k, n)
    ref = synth.to_f32(xi, synth.BF16).astype(np.int64) @ \
        synth.to_f32(wi, synth.BF16).astype(np.int64).T + synth.to_f32(bi, synth.BF16).astype(np.int64)
    assert np.array_equal(r.out, _bf16(ref.astype(np.float32)))


def test_fp8_linear_backward_vs_numpy():
    m, k, n = 41, 70, 53
    g = synth.normal_bits((m, n), 1.0, 6, 1, synth.BF16)
    x = synth.normal_bits((m, k), 1.0, 6, 2, synth.BF16)
    w = synth.normal_bits((n, k), 0.5, 6, 3, synth.BF16)
    sg_inv, sw_inv, sx_inv = 100.0, 150.0, 90.0
    sg, sw, sx = 1 / sg_inv, 1 / sw_inv, 1 / sx_inv
    f = lambda v: float(np.float32(v))
    rdx = oracle.fp8_linear_backward("dx", g, x, w, sg, sw, sx, sg_inv, sw_inv, sx_inv, m, k, n)
    rdw = oracle.fp8_linear_backward("dw", g, x, w, sg, sw, sx, sg_inv, sw_inv, sx_inv, m, k, n)
    qg, qw, qx = _torch_quant(g, sg_inv), _torch_quant(w, sw_inv), _torch_quant(x, sx_inv)
    assert np.allclose(rdx.s, (qg @ qw) * f(sg) * f(sw), rtol=1e-12, atol=1e-12)
    assert np.allclose(rdw.s, (qg.T @ qx) * f(sg) * f(sx), rtol=1e-12, atol=1e-12)
    assert rdx.amax_g == np.abs(synth.to_f32(g, synth.BF16)).max()
    # row selection gives the same rows
    sel = oracle.fp8_linear_backward("dw", g, x, w, sg, sw, sx, sg_inv, sw_inv, sx_inv, m, k, n,
                                     rows=[0, 17, 52])
    assert np.array_equal(sel.out, rdw.out[[0, 17, 52]])


def test_fp8_group_max_statistic_by_hand():
    # one output element, reduction of 10: products 1..10 (a = 1..10 as e4m3
    # codes of exact small integers, b = 1): groups {0..7} and {8, 9} have
    # maxima 8 and 10, so G = 18; with scales 0.5 and 0.25, G = 18 / 8
    vals = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10]
    a8 = np.array([[oracle.rne_e4m3_sat(v) for v in vals]], np.uint8)
    bt8 = np.array([[oracle.rne_e4m3_sat(1.0)] * 10], np.uint8)
    r = oracle.fp8_mm(a8, bt8, 0.5, 0.25, 1, 10, 1)
    assert r.g[0, 0] == 18 / 8 and r.s[0, 0] == 55 / 8
    # the same statistic from the fp8 linear (negative products count by size)
    x = _bf16([[1, -2, 3, -4, 5, -6, 7, -8, 9, -10]])
    w = _bf16([[1] * 10])
    f = oracle.fp8_linear_forward(x, w, None, 1.0, 1.0, 1.0, 1.0, 1, 10, 1)
    assert f.g[0, 0] == 18 and f.s[0, 0] == -5


@pytest.mark.parametrize("dt", [synth.F32, synth.BF16, synth.F16])
def test_bias_grad_vs_numpy_column_sum(dt):
    m, n = 333, 77
    dy = synth.normal_bits((m, n), 1.0, 8, 4, dt)
    r = oracle.bias_grad(dt, dy, m, n)
    v = synth.to_f32(dy, dt).astype(np.float64)
    # sums of at most a few hundred values of <= 24 significant bits in
    # double are exact, so numpy's pairwise sum is the same number
    assert np.array_equal(r.s, v.sum(axis=0))
    assert np.array_equal(r.a, np.abs(v).sum(axis=0))
    ref = torch.from_numpy(v.sum(axis=0)).to({synth.F32: torch.float32,
                                               synth.BF16: torch.bfloat16,
                                               synth.F16: torch.float16}[dt])
    bits = ref.view({synth.F32: torch.int32, synth.BF16: torch.int16,
                     synth.F16: torch.int16}[dt]).numpy()
    assert np.array_equal(r.out.view(bits.dtype), bits)
