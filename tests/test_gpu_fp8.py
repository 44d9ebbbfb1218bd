"""GPU parity of the per-tensor-scaled fp8 e4m3 GEMM against the CPU oracle,
with the determinism contracts (run-to-run hashes, batch invariance).

The default MFMA path (tc = 1) widens every e4m3 code exactly to bf16 and adds
the exact products with the bf16 matrix instruction at f32 precision (AstrAI
fp8_mm.cu, fp8_gemm_into: f32 compute type), so it meets the plain rule of
tests/parity.py (1 ulp of bf16, or 1e-5 of sum |a*b|).  The opt-in fast path
(tc = 3, the fp8 matrix instruction) is checked with its own wider rule, and its
distance from the plain rule is asserted as measured."""
import numpy as np
import pytest
import torch

import deterministic_invariant_gemm_amd as dig
import oracle
import synth
from parity import check, dev, digest, empty, f32_scalar, group_stats, host, sample_rows

pytestmark = pytest.mark.gpu

FAST = dig.TC_FP8_FAST


class Fp8:
    def __init__(self, d):
        self.d = d
        self.m, self.k, self.n = d["m"], d["k"], d["n"]
        self.a, self.bt = dev(d["a8"]), dev(d["bt8"])
        self.da, self.db = f32_scalar(float(d["da"])), f32_scalar(float(d["db"]))

    def run(self, tc, m=None):
        m = self.m if m is None else m
        y = empty((m, self.n), np.uint16)
        dig.check(dig.bi_fp8_mm(y, self.a, self.bt, self.da, self.db, m, self.k, self.n,
                                torch.cuda.current_stream(), tc), "bi_fp8_mm")
        return y


def test_e4m3_format_is_ocp():
    """Code 0x7E must act as 448 (OCP e4m3fn), not 224 (the FNUZ flavour):
    A = [[448]*64], B^T = [[1]*64] gives 64*448 = 28672 exactly."""
    k = 64
    for tc in (0, 1, FAST):
        d = {"a8": np.full((64, k), 0x7E, np.uint8), "bt8": np.full((64, k), 0x38, np.uint8),
             "da": np.float32(1.0), "db": np.float32(1.0), "m": 64, "k": k, "n": 64}
        y = host(Fp8(d).run(tc), np.uint16)
        assert np.all(y == synth.to_bits(np.array([28672.0], np.float32), synth.BF16)[0]), tc


@pytest.mark.parametrize("tc", [0, 1, FAST])
@pytest.mark.parametrize("shape", [(300, 256, 260), (129, 200, 96), (1, 64, 64),
                                   (70, 1000, 130), (5, 7, 3), (300, 1008, 48)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp8_parity_small(tc, shape):
    m, k, n = shape
    d = synth.fp8(m, k, n, seed=200 + m + k)
    print(f"fp8 parity tc={tc} shape={shape}", flush=True)
    r = oracle.fp8_mm(d["a8"], d["bt8"], d["da"], d["db"], m, k, n)
    check(host(Fp8(d).run(tc), np.uint16), r, synth.BF16, f"fp8 {shape}", groups=tc == FAST)


@pytest.mark.parametrize("tc", [0, 1, FAST])
@pytest.mark.parametrize("shape", [(300, 256, 260), (70, 1000, 130), (257, 4096, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp8_exact_integer_bits(tc, shape):
    """Integer e4m3 codes in [-8, 8] with power-of-two scales: exact in any
    summation order, so the GPU must equal the oracle bit for bit."""
    m, k, n = shape
    d = synth.fp8_integer(m, k, n, seed=9)
    r = oracle.fp8_mm(d["a8"], d["bt8"], d["da"], d["db"], m, k, n)
    assert np.array_equal(host(Fp8(d).run(tc), np.uint16), r.out)


def test_fp8_8192x4096x4096():
    """A[8192,4096], B^T[4096,4096] quantised from N(0,1) bf16 with scale
    448/amax, default path: the plain rule on 259 sampled rows at M = 8192
    and on every element at M = 16 (the first 16 rows), 10-run hashes at both
    sizes and batch invariance between them."""
    d = synth.fp8_8192x4096x4096()
    F = Fp8(d)
    m, k, n = F.m, F.k, F.n
    y = host(F.run(1), np.uint16)
    rows = sample_rows(m, 256, 6)
    assert len(rows) >= 256
    r = oracle.fp8_mm(d["a8"], d["bt8"], d["da"], d["db"], m, k, n, rows=rows)
    print("fp8_8192x4096x4096 M=8192 (max ulp, #>1 ulp, max rel):",
          check(y[rows], r, synth.BF16, "fp8_8192x4096x4096 M=8192"))
    y16 = host(F.run(1, m=16), np.uint16)
    r16 = oracle.fp8_mm(d["a8"], d["bt8"], d["da"], d["db"], m, k, n, rows=np.arange(16))
    print("fp8_8192x4096x4096 M=16:", check(y16, r16, synth.BF16, "fp8_8192x4096x4096 M=16"))
    assert np.array_equal(y16, y[:16])
    assert len({digest(F.run(1)) for _ in range(10)}) == 1
    assert len({digest(F.run(1, m=16)) for _ in range(10)}) == 1


# the fast path's distance from the plain rule on the 8192x4096x4096 workload
# (its bits are deterministic, so these are exact measured values): at M = 16
# (every element) and on the sampled rows at M = 8192
FAST_STATS_M16 = (30, 80, 0)
FAST_STATS_M8192 = (29897, 1261, 0)


def test_fp8_fast_8192x4096x4096():
    """The opt-in fast path on the same workload: its own rule (2^-10 G added),
    its measured max ulp and the count of elements that pass only through the
    G clause asserted, 10-run hashes and batch invariance."""
    d = synth.fp8_8192x4096x4096()
    F = Fp8(d)
    m, k, n = F.m, F.k, F.n
    y = host(F.run(FAST), np.uint16)
    rows = sample_rows(m, 256, 6)
    r = oracle.fp8_mm(d["a8"], d["bt8"], d["da"], d["db"], m, k, n, rows=rows)
    check(y[rows], r, synth.BF16, "fast fp8 M=8192", groups=True)
    s8192 = group_stats(y[rows], r, synth.BF16)
    y16 = host(F.run(FAST, m=16), np.uint16)
    r16 = oracle.fp8_mm(d["a8"], d["bt8"], d["da"], d["db"], m, k, n, rows=np.arange(16))
    check(y16, r16, synth.BF16, "fast fp8 M=16", groups=True)
    s16 = group_stats(y16, r16, synth.BF16)
    print("fast fp8 (max ulp, #>1 ulp, #needing G): M=16", s16, "M=8192 rows", s8192)
    assert s16 == FAST_STATS_M16
    assert s8192 == FAST_STATS_M8192
    assert np.array_equal(y16, y[:16])
    assert len({digest(F.run(FAST)) for _ in range(10)}) == 1


def _one_product_row(terms, K, tc):
    """a [1,K], b^T [64,K] e4m3 codes with a[j], b[:, j] from (j, a, b) terms."""
    a = np.zeros((1, K), np.uint8)
    b = np.zeros((64, K), np.uint8)
    for j, av, bv in terms:
        a[0, j] = oracle.rne_e4m3_sat(av)
        b[:, j] = oracle.rne_e4m3_sat(bv)
    y = empty((1, 64), np.uint16)
    one = f32_scalar(1.0)
    dig.check(dig.bi_fp8_mm(y, dev(a), dev(b), one, one, 1, K, 64,
                            torch.cuda.current_stream(), tc), "bi_fp8_mm")
    return oracle.decode_bf16(int(host(y, np.uint16)[0, 0]))


def test_fp8_default_adds_exact_products():
    """The default path keeps what the fp8 matrix instruction drops: small
    products beside a large one inside one 16-deep step (1 + 2^-18 - 1), two
    halves of an f32 ulp that sequential f32 addition would round away
    (2^12 + 2^-12 + 2^-12 = 2^12 + 2^-11), and the same across steps."""
    assert _one_product_row([(0, 1.0, 1.0), (3, 2.0 ** -9, 2.0 ** -9), (10, 1.0, -1.0)],
                            64, 1) == 2.0 ** -18
    assert _one_product_row([(0, 1.0, 1.0), (1, 2.0 ** -7, 2.0 ** -7), (2, 1.0, -1.0)],
                            64, 1) == 2.0 ** -14
    assert _one_product_row([(0, 64.0, 64.0), (5, 2.0 ** -6, 2.0 ** -6),
                             (6, 2.0 ** -6, 2.0 ** -6), (40, 64.0, -64.0)], 64, 1) == 2.0 ** -11
    assert _one_product_row([(0, 1.0, 1.0), (17, 2.0 ** -9, 2.0 ** -9), (33, 1.0, -1.0)],
                            64, 1) == 2.0 ** -18


def test_fp8_fast_group_alignment():
    """The behaviour of the fp8 matrix instruction that the fast path's rule
    rests on: within one 64-deep step, products are added in groups of 8
    consecutive reduction indices aligned to the group's largest product with
    13 bits below it; the accumulator across steps is f32."""
    # in the 1's group of 8: 1 + 2^-13 - 1 keeps the small product, 1 + 2^-14 - 1
    # loses it
    assert _one_product_row([(0, 1.0, 1.0), (3, 2.0 ** -7, 2.0 ** -6), (20, 1.0, -1.0)],
                            64, FAST) == 2.0 ** -13
    assert _one_product_row([(0, 1.0, 1.0), (3, 2.0 ** -7, 2.0 ** -7), (20, 1.0, -1.0)],
                            64, FAST) == 0.0
    # in another group of the same step it is kept (index 9: group 8..15)
    assert _one_product_row([(0, 1.0, 1.0), (9, 2.0 ** -7, 2.0 ** -7), (20, 1.0, -1.0)],
                            64, FAST) == 2.0 ** -14
    # across steps the running f32 sum keeps it
    assert _one_product_row([(0, 1.0, 1.0), (64 + 9, 2.0 ** -9, 2.0 ** -9),
                             (128 + 3, 1.0, -1.0)], 192, FAST) == 2.0 ** -18
    # 63 products of 2^-15 beside a 1 in the same step: only the 7 sharing the
    # 1's group of 8 are lost
    terms = [(0, 1.0, 1.0)] + [(j, 2.0 ** -7, 2.0 ** -8) for j in range(1, 64)]
    assert _one_product_row(terms + [(64, 1.0, -1.0)], 128, FAST) == 56 * 2.0 ** -15
