"""GPU parity of the fp8 producer side against the CPU oracle: quantisation
and transposed quantisation (bit-exact codes and amax, e4m3fn and e5m2), and
the scaled fp8 linear forward / backward (the pass rule of the fp8 GEMM;
bit-exact on integer data, where every step is exact)."""
import numpy as np
import pytest
import torch

import deterministic_invariant_gemm_amd as dig
import oracle
import synth
from parity import check, dev, digest, empty, f32_scalar, host, sample_rows

pytestmark = pytest.mark.gpu

FMTS = {"e4m3": (dig.BI_FP8_E4M3, oracle.E4M3), "e5m2": (dig.BI_FP8_E5M2, oracle.E5M2)}


def edge_values(fmt_max):
    """bf16 sources that, times the scales used below, land on subnormals,
    exact codes, ties between codes, the largest finite value, beyond it, and
    the signed zeros and infinities."""
    v = [0.0, -0.0, 1.0, -1.0, 1.0625, 1.1875, -1.0625, 3.0, 2.0 ** -9, 2.0 ** -10,
         1.5 * 2.0 ** -10, 2.0 ** -16, 1.5 * 2.0 ** -16, 2.0 ** -17, fmt_max, fmt_max * 1.02,
         fmt_max * 1.2, -fmt_max * 1.5, 1e30, -1e30, float("inf"), float("-inf")]
    return synth.to_bits(np.array(v, dtype=np.float32), synth.BF16)


def gpu_quantize(src_bits, scale_inv, fmt, offset=0, amax0=0.0):
    n = src_bits.size
    # `offset` elements of padding in front make the buffers misaligned
    src = dev(np.concatenate([np.zeros(offset, np.uint16), src_bits.ravel()]))
    dst = empty(n + offset, np.uint8)
    amax = f32_scalar(amax0)
    si = f32_scalar(scale_inv)
    dig.check(dig.bi_fp8_quantize(dst[offset:], src[offset:], si, amax, n, fmt,
                                  torch.cuda.current_stream()), "bi_fp8_quantize")
    return host(dst, np.uint8)[offset:], float(host(amax, np.float32)[0])


@pytest.mark.parametrize("fmt", sorted(FMTS))
@pytest.mark.parametrize("n,offset", [(1, 0), (15, 0), (16, 0), (17, 0), (1000003, 0),
                                      (4099, 1), (70000, 3)])
def test_quantize_bit_exact(fmt, n, offset):
    gfmt, ofmt = FMTS[fmt]
    mx = 448.0 if fmt == "e4m3" else 57344.0
    g = np.random.default_rng(n + offset)
    # normal data spread over the whole format range, plus the edge values
    f = (g.standard_normal(n) * np.exp2(g.integers(-12, 12, n))).astype(np.float32)
    src = synth.to_bits(f, synth.BF16)
    e = edge_values(mx)
    src[:min(n, e.size)] = e[:min(n, e.size)]
    for scale_inv in (1.0, 0.75, 37.5):
        got, amax = gpu_quantize(src, scale_inv, gfmt, offset)
        ref, ramax = oracle.fp8_quantize(ofmt, src, scale_inv)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (fmt, scale_inv, [(int(i), int(src[i]), int(got[i]), int(ref[i]))
                                                for i in bad[:8]])
        assert amax == ramax, (amax, ramax)


def test_quantize_amax_folds_into_existing_value():
    src = synth.to_bits(np.array([1.0, -3.0, 2.0], np.float32), synth.BF16)
    _, a = gpu_quantize(src, 1.0, dig.BI_FP8_E4M3, amax0=0.0)
    assert a == 3.0
    _, a = gpu_quantize(src, 1.0, dig.BI_FP8_E4M3, amax0=7.5)
    assert a == 7.5


@pytest.mark.parametrize("fmt", sorted(FMTS))
@pytest.mark.parametrize("rows,cols", [(1, 1), (64, 64), (100, 72), (130, 200), (77, 33),
                                       (4096, 768), (16, 4096)])
def test_transpose_quantize_bit_exact(fmt, rows, cols):
    gfmt, ofmt = FMTS[fmt]
    g = np.random.default_rng(rows * 7 + cols)
    f = (g.standard_normal((rows, cols)) * np.exp2(g.integers(-8, 8, (rows, cols)))).astype(np.float32)
    src = synth.to_bits(f, synth.BF16)
    d_src = dev(src)
    dst = empty(rows * cols, np.uint8)
    amax = f32_scalar(0.0)
    dig.check(dig.bi_fp8_transpose_quantize(dst, d_src, f32_scalar(3.0), amax, rows, cols, gfmt,
                                            torch.cuda.current_stream()), "transpose_quantize")
    ref, ramax = oracle.fp8_transpose_quantize(ofmt, src, 3.0, rows, cols)
    assert np.array_equal(host(dst, np.uint8).reshape(cols, rows), ref)
    assert float(host(amax, np.float32)[0]) == ramax


class Fp8Linear:
    def __init__(self, d):
        self.d = d
        self.m, self.k, self.n = d["m"], d["k"], d["n"]
        self.x, self.w, self.g = dev(d["x"]), dev(d["w"]), dev(d["g"])
        self.b = dev(d["b"]) if d["b"] is not None else None
        self.sc = {k: f32_scalar(float(d[k])) for k in
                   ("sx", "sw", "sg", "sx_inv", "sw_inv", "sg_inv")}
        nb = dig.bi_fp8_linear_workspace_bytes(self.m, self.k, self.n)
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        self.ws.fill_(77)
        self.nb = nb

    def forward(self, tc=1):
        y = empty((self.m, self.n), np.uint16)
        ax, aw = f32_scalar(-1.0), f32_scalar(-1.0)
        c = self.sc
        dig.check(dig.bi_fp8_linear_forward(y, self.x, self.w, self.b, c["sx"], c["sw"],
                                            c["sx_inv"], c["sw_inv"], ax, aw, self.m, self.k,
                                            self.n, self.ws, self.nb,
                                            torch.cuda.current_stream(), tc), "fp8 forward")
        return y, float(host(ax, np.float32)[0]), float(host(aw, np.float32)[0])

    def backward(self, want_dx=True, want_dw=True, tc=1):
        dx = empty((self.m, self.k), np.uint16) if want_dx else None
        dw = empty((self.n, self.k), np.uint16) if want_dw else None
        ag = f32_scalar(-1.0)
        c = self.sc
        dig.check(dig.bi_fp8_linear_backward(dx, dw, self.g, self.x, self.w, c["sg"], c["sw"],
                                             c["sx"], c["sg_inv"], c["sw_inv"], c["sx_inv"], ag,
                                             self.m, self.k, self.n, self.ws, self.nb,
                                             torch.cuda.current_stream(), tc), "fp8 backward")
        return dx, dw, float(host(ag, np.float32)[0])


def oracle_args(d):
    return (d["sx"], d["sw"], d["sx_inv"], d["sw_inv"])


@pytest.mark.parametrize("tc", [0, 1, 3])
@pytest.mark.parametrize("shape,bias", [((300, 256, 260), True), ((129, 200, 96), False),
                                        ((1, 64, 64), True), ((520, 384, 392), True)],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_fp8_linear_parity(shape, bias, tc):
    m, k, n = shape
    d = synth.fp8_linear(m, k, n, seed=300 + m, bias=bias)
    L = Fp8Linear(d)
    y, ax, aw = L.forward(tc)
    r = oracle.fp8_linear_forward(d["x"], d["w"], d["b"], *oracle_args(d), m, k, n)
    check(host(y, np.uint16), r, synth.BF16, f"fp8 linear forward {shape}", groups=tc == 3)
    assert (ax, aw) == (r.amax_x, r.amax_w)
    dx, dw, ag = L.backward(tc=tc)
    args = (d["g"], d["x"], d["w"], d["sg"], d["sw"], d["sx"], d["sg_inv"], d["sw_inv"],
            d["sx_inv"], m, k, n)
    rdx = oracle.fp8_linear_backward("dx", *args)
    rdw = oracle.fp8_linear_backward("dw", *args)
    check(host(dx, np.uint16), rdx, synth.BF16, f"fp8 linear dX {shape}", groups=tc == 3)
    check(host(dw, np.uint16), rdw, synth.BF16, f"fp8 linear dW {shape}", groups=tc == 3)
    assert ag == rdx.amax_g
    # one gradient at a time gives the same bits
    dx1, dw1, ag1 = L.backward(want_dw=False, tc=tc)
    dx2, dw2, ag2 = L.backward(want_dx=False, tc=tc)
    assert dw1 is None and dx2 is None
    assert digest(dx1) == digest(dx) and digest(dw2) == digest(dw)
    assert ag1 == ag2 == rdx.amax_g


def test_fp8_linear_integer_bit_exact():
    """Integer sources in [-6, 6] with unit scales: quantisation, products,
    sums and scaling are all exact, so every output bit is fixed."""
    m, k, n = 257, 512, 200
    g = np.random.default_rng(9)
    ints = lambda shape: synth.to_bits(g.integers(-6, 7, shape).astype(np.float32), synth.BF16)
    d = {"x": ints((m, k)), "w": ints((n, k)), "g": ints((m, n)), "b": ints((n,)),
         "m": m, "k": k, "n": n}
    for s in ("x", "w", "g"):
        d["s" + s] = np.float32(1.0)
        d["s" + s + "_inv"] = np.float32(1.0)
    L = Fp8Linear(d)
    y, _, _ = L.forward()
    r = oracle.fp8_linear_forward(d["x"], d["w"], d["b"], 1.0, 1.0, 1.0, 1.0, m, k, n)
    assert np.array_equal(host(y, np.uint16), r.out)
    dx, dw, _ = L.backward()
    args = (d["g"], d["x"], d["w"], 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, m, k, n)
    assert np.array_equal(host(dx, np.uint16), oracle.fp8_linear_backward("dx", *args).out)
    assert np.array_equal(host(dw, np.uint16), oracle.fp8_linear_backward("dw", *args).out)


def test_fp8_linear_config_sampled_and_deterministic():
    """x [4096,4096], w [4096,4096], g [4096,4096]: sampled rows against the
    oracle, and the same bytes on every run."""
    m = k = n = 4096
    d = synth.fp8_linear(m, k, n, seed=44)
    L = Fp8Linear(d)
    y, _, _ = L.forward()
    dx, dw, _ = L.backward()
    rows = sample_rows(m, 12, 1)
    r = oracle.fp8_linear_forward(d["x"], d["w"], d["b"], *oracle_args(d), m, k, n, rows=rows)
    check(host(y, np.uint16)[rows], r, synth.BF16, "fp8 linear forward 4096")
    args = (d["g"], d["x"], d["w"], d["sg"], d["sw"], d["sx"], d["sg_inv"], d["sw_inv"],
            d["sx_inv"], m, k, n)
    check(host(dx, np.uint16)[rows], oracle.fp8_linear_backward("dx", *args, rows=rows),
          synth.BF16, "fp8 linear dX 4096")
    check(host(dw, np.uint16)[rows], oracle.fp8_linear_backward("dw", *args, rows=rows),
          synth.BF16, "fp8 linear dW 4096")
    hy, hdx, hdw = digest(y), digest(dx), digest(dw)
    for _ in range(3):
        y2, _, _ = L.forward()
        dx2, dw2, _ = L.backward()
        assert (digest(y2), digest(dx2), digest(dw2)) == (hy, hdx, hdw)
