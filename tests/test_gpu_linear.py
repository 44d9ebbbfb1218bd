"""GPU parity of the linear trio (forward, dX, dW) against the CPU oracle,
plus the determinism contracts: run-to-run byte equality, batch invariance of
the forward, identical bits across tile shapes, and the scalar tier's
bf16/f16 == RNE(f32 tier on upcast inputs) statement."""
import numpy as np
import pytest
import torch

import deterministic_invariant_gemm_amd as dig
import oracle
import synth
from parity import check, dev, digest, empty, host, sample_rows

pytestmark = pytest.mark.gpu

ST = {synth.F32: np.uint32, synth.BF16: np.uint16, synth.F16: np.uint16}


class Linear:
    """Device copies of one linear workload and calls through the C ABI."""

    def __init__(self, d):
        self.d = d
        self.m, self.k, self.n, self.dt = d["m"], d["k"], d["n"], d["dt"]
        self.st = ST[self.dt]
        self.x, self.w, self.dy = dev(d["x"]), dev(d["w"]), dev(d["dy"])
        self.b = dev(d["b"]) if d["b"] is not None else None

    def forward(self, tc, m=None):
        m = self.m if m is None else m
        y = empty((m, self.n), self.st)
        dig.check(dig.bi_forward(y, self.x, self.w, self.b, m, self.k, self.n, self.dt,
                                 torch.cuda.current_stream(), tc), "bi_forward")
        return y

    def dx(self, tc, m=None):
        m = self.m if m is None else m
        out = empty((m, self.k), self.st)
        dig.check(dig.bi_backward_dx(out, self.dy, self.w, m, self.k, self.n, self.dt,
                                     torch.cuda.current_stream(), tc), "bi_backward_dx")
        return out

    def dw(self, tc):
        out = empty((self.k, self.n), self.st)
        nbytes = dig.bi_backward_dw_workspace_bytes(self.m, self.k, self.n, self.dt, tc)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        ws.fill_(255)
        dig.check(dig.bi_backward_dw(out, self.x, self.dy, self.m, self.k, self.n, self.dt,
                                     ws if nbytes else None, nbytes,
                                     torch.cuda.current_stream(), tc), "bi_backward_dw")
        return out


def full_parity(d, tc, what):
    L = Linear(d)
    m, k, n, dt = L.m, L.k, L.n, L.dt
    ry = oracle.linear_forward(dt, d["x"], d["w"], d["b"], m, k, n)
    check(host(L.forward(tc), L.st), ry, dt, f"{what} fwd")
    rx = oracle.linear_dx(dt, d["dy"], d["w"], m, k, n)
    check(host(L.dx(tc), L.st), rx, dt, f"{what} dX")
    rw = oracle.linear_dw(dt, d["x"], d["dy"], m, k, n)
    check(host(L.dw(tc), L.st), rw, dt, f"{what} dW")


# shapes spanning several tiles of every tier, with ragged tails in every dim
SHAPES = [(300, 200, 260), (129, 72, 96), (1, 64, 64), (257, 1000, 130), (70, 136, 72),
          (64, 33, 65), (5, 7, 3)]


@pytest.mark.parametrize("dt", [synth.F32, synth.BF16, synth.F16])
@pytest.mark.parametrize("tc", [0, 1])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_linear_parity_small(dt, tc, shape):
    m, k, n = shape
    d = synth.linear(m, k, n, dt, seed=100 + m + k + n, sigma_w=0.05)
    print(f"linear parity dt={dt} tc={tc} shape={shape}", flush=True)
    full_parity(d, tc, f"dt{dt} tc{tc} {shape}")


# outputs of at most 64 columns run the scalar tier's one-row-per-lane kernel:
# whole and partial reduction slices, 16-byte and one-value loads of A (odd K),
# one column, a dW reduced over three 256-row chunks (M = 700)
NARROW = [(300, 1000, 48), (257, 256, 1), (65, 520, 63), (1, 384, 17), (700, 136, 40),
          (130, 301, 48), (300, 48, 1000), (129, 40, 136), (2000, 64, 33), (70, 17, 200)]


@pytest.mark.parametrize("dt", [synth.F32, synth.BF16, synth.F16])
@pytest.mark.parametrize("shape", NARROW, ids=lambda s: "x".join(map(str, s)))
def test_linear_parity_narrow(dt, shape):
    m, k, n = shape
    d = synth.linear(m, k, n, dt, seed=300 + m + k + n, sigma_w=0.05)
    print(f"narrow linear parity dt={dt} shape={shape}", flush=True)
    full_parity(d, 0, f"narrow dt{dt} {shape}")


@pytest.mark.parametrize("dt", [synth.BF16, synth.F16, synth.F32])
@pytest.mark.parametrize("tc", [0, 1])
@pytest.mark.parametrize("shape", [(300, 200, 260), (257, 1000, 130), (4100, 96, 72),
                                   (33, 4096, 64)], ids=lambda s: "x".join(map(str, s)))
def test_linear_exact_integer_bits(dt, tc, shape):
    """Small-integer operands: every partial sum is an exactly representable
    integer, so f32 accumulation is exact in any order and every tier, tile,
    chunking and layout must reproduce the oracle bit for bit."""
    m, k, n = shape
    d = synth.linear_integer(m, k, n, dt, seed=7 + m, lo=-3, hi=3)
    L = Linear(d)
    print(f"exact integer dt={dt} tc={tc} shape={shape}", flush=True)
    ry = oracle.linear_forward(dt, d["x"], d["w"], d["b"], m, k, n)
    assert np.array_equal(host(L.forward(tc), L.st), ry.out)
    rx = oracle.linear_dx(dt, d["dy"], d["w"], m, k, n)
    assert np.array_equal(host(L.dx(tc), L.st), rx.out)
    rw = oracle.linear_dw(dt, d["x"], d["dy"], m, k, n)
    assert np.array_equal(host(L.dw(tc), L.st), rw.out)


def test_f32_linear_64x128x256():
    """f32 X[64,128] W[128,256] + b, dY[64,256]: parity, 10-run hashes and batch
    invariance at M' in {1, 7, 64}."""
    d = synth.f32_linear_64x128x256()
    full_parity(d, 1, "f32_linear_64x128x256")
    L = Linear(d)
    for op in (lambda: L.forward(1), lambda: L.dx(1), lambda: L.dw(1)):
        assert len({digest(op()) for _ in range(10)}) == 1
    y = host(L.forward(1), np.uint32)
    for mp in (1, 7, 64):
        assert np.array_equal(host(L.forward(1, m=mp), np.uint32), y[:mp])


def linear_backward(L, tc=1):
    """dX and dW from one bi_linear_backward call (its dX and dW tiles share a
    launch at 4096x768x3072)."""
    m, k, n, dt = L.m, L.k, L.n, L.dt
    dx, dw = empty((m, k), L.st), empty((k, n), L.st)
    nb = dig.bi_backward_dw_workspace_bytes(m, k, n, dt, tc)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    dig.check(dig.bi_linear_backward(dx, dw, L.dy, L.x, L.w, m, k, n, dt, ws if nb else None,
                                     nb, torch.cuda.current_stream(), tc), "bi_linear_backward")
    return dx, dw


@pytest.mark.parametrize("dt", [synth.BF16, synth.F16])
def test_mlp_up_parity_full(dt):
    """X[4096,768] W[768,3072] + b, dY[4096,3072] on the MFMA tier: every
    element of the forward, dX and dW against the oracle, from the separate
    calls and from bi_linear_backward (whose bits must equal the separate
    calls')."""
    d = synth.mlp_up_linear(dt)
    L = Linear(d)
    m, k, n = L.m, L.k, L.n
    stats = {}
    y = host(L.forward(1), L.st)
    stats["fwd"] = check(y, oracle.linear_forward(dt, d["x"], d["w"], d["b"], m, k, n), dt,
                         "mlp_up_linear fwd")
    dx, dw = host(L.dx(1), L.st), host(L.dw(1), L.st)
    stats["dX"] = check(dx, oracle.linear_dx(dt, d["dy"], d["w"], m, k, n), dt,
                        "mlp_up_linear dX")
    stats["dW"] = check(dw, oracle.linear_dw(dt, d["x"], d["dy"], m, k, n), dt,
                        "mlp_up_linear dW")
    bx, bw = linear_backward(L)
    assert np.array_equal(host(bx, L.st), dx) and np.array_equal(host(bw, L.st), dw)
    print("mlp_up_linear (max ulp, #beyond 1 ulp, max rel):", stats)


@pytest.mark.parametrize("dt", [synth.BF16, synth.F16])
def test_mlp_up_exact_integer_bits(dt):
    """4096x768x3072 with integers in [-3, 3]: every partial sum is exact in
    f32 (|sum| <= 4096 * 9 < 2^24), so the production tiles (the forward's
    256x192 tile, dX 128x96 and dW 96x96 alone and sharing one launch) must
    reproduce the oracle bit for bit in every element."""
    m, k, n = 4096, 768, 3072
    d = synth.linear_integer(m, k, n, dt, seed=17, lo=-3, hi=3)
    L = Linear(d)
    assert np.array_equal(host(L.forward(1), L.st),
                          oracle.linear_forward(dt, d["x"], d["w"], d["b"], m, k, n).out)
    rx = oracle.linear_dx(dt, d["dy"], d["w"], m, k, n).out
    rw = oracle.linear_dw(dt, d["x"], d["dy"], m, k, n).out
    assert np.array_equal(host(L.dx(1), L.st), rx)
    assert np.array_equal(host(L.dw(1), L.st), rw)
    bx, bw = linear_backward(L)
    assert np.array_equal(host(bx, L.st), rx) and np.array_equal(host(bw, L.st), rw)


# M' for the batch-invariance check at K = 768, N = 3072.  The forward runs
# the 256x192 tile from M' = 2817 (at least 192 workgroups), the 128x128 tile
# for 897..2816, and the 64x32 tile up to M' = 128 (one round of at most 256
# workgroups); dX (768 output columns) runs the 64x32 tile up to M' = 640 and
# the 128x96 tile beyond.  The list covers every one of these tiles.
MLP_UP_MPRIME = (1, 7, 64, 100, 128, 640, 1000, 2000, 2816, 3000, 4096)


@pytest.mark.parametrize("dt", [synth.BF16, synth.F16])
def test_mlp_up_determinism_and_batch_invariance(dt):
    d = synth.mlp_up_linear(dt)
    L = Linear(d)
    for name, op in (("fwd", lambda: L.forward(1)), ("dX", lambda: L.dx(1)),
                     ("dW", lambda: L.dw(1)),
                     ("bi_linear_backward", lambda: torch.cat([t.flatten() for t in
                                                               linear_backward(L)]))):
        assert len({digest(op()) for _ in range(10)}) == 1, name
    y = host(L.forward(1), np.uint16)
    dx = host(L.dx(1), np.uint16)
    for mp in MLP_UP_MPRIME:
        assert np.array_equal(host(L.forward(1, m=mp), np.uint16), y[:mp]), mp
        assert np.array_equal(host(L.dx(1, m=mp), np.uint16), dx[:mp]), mp


def test_mlp_up_narrow_n48():
    """N = 48 < 64: forward and dW fall back to the scalar tier, dX (output dim
    K = 768) stays on MFMA; sampled parity and run-to-run hashes."""
    d = synth.mlp_up_linear(synth.BF16, n=48, seed=22)
    L = Linear(d)
    m, k, n, dt = L.m, L.k, L.n, L.dt
    assert dig.bi_plan(dig.OP_FWD, dt, 1, k, n)[0] == 0
    assert dig.bi_plan(dig.OP_DW, dt, 1, k, n)[0] == 0
    assert dig.bi_plan(dig.OP_DX, dt, 1, k, n)[0] > 0
    rows = sample_rows(m, 64, 3)
    ry = oracle.linear_forward(dt, d["x"], d["w"], d["b"], m, k, n, rows=rows)
    check(host(L.forward(1), L.st)[rows], ry, dt, "n48 fwd")
    rx = oracle.linear_dx(dt, d["dy"], d["w"], m, k, n, rows=rows)
    check(host(L.dx(1), L.st)[rows], rx, dt, "n48 dX")
    rw = oracle.linear_dw(dt, d["x"], d["dy"], m, k, n)
    check(host(L.dw(1), L.st), rw, dt, "n48 dW")
    for op in (lambda: L.forward(1), lambda: L.dx(1), lambda: L.dw(1)):
        assert len({digest(op()) for _ in range(10)}) == 1
    y = host(L.forward(1), np.uint16)
    for mp in (1, 7, 64):
        assert np.array_equal(host(L.forward(1, m=mp), np.uint16), y[:mp])


def test_scalar_tier_bf16_is_rne_of_f32_on_upcast():
    """Scalar-tier contract: the bf16 (and f16) result equals the f32 tier run on
    the exactly upcast inputs, then rounded once to nearest-even."""
    for dt, (m, k, n) in ((synth.BF16, (130, 300, 70)), (synth.F16, (130, 300, 70)),
                          (synth.BF16, (700, 520, 40)), (synth.F16, (700, 520, 40))):
        d = synth.linear(m, k, n, dt, seed=31, sigma_w=0.05)
        up = dict(d)
        for t in ("x", "w", "b", "dy"):
            up[t] = synth.to_bits(synth.to_f32(d[t], dt), synth.F32)
        up["dt"] = synth.F32
        Lb, Lf = Linear(d), Linear(up)
        for name in ("forward", "dx", "dw"):
            low = host(getattr(Lb, name)(0), np.uint16)
            f32 = host(getattr(Lf, name)(0), np.uint32).view(np.float32)
            assert np.array_equal(low, synth.to_bits(f32, dt)), (dt, (m, k, n), name)


def test_tile_families_give_identical_bits():
    """The same output columns computed under different tile shapes (the plan
    picks the tile from N) are bit-identical."""
    dt = synth.BF16
    m, k = 600, 512
    d = synth.linear(m, k, 4096, dt, seed=41, sigma_w=0.02)
    full = Linear(d)
    y_full = host(full.forward(1), np.uint16)
    tiles = {dig.bi_plan(dig.OP_FWD, dt, 1, k, 4096)[0]}
    for n in (3072, 384, 96):
        sub = dict(d)
        sub["w"] = np.ascontiguousarray(d["w"][:, :n])
        sub["b"] = np.ascontiguousarray(d["b"][:n])
        sub["dy"] = np.ascontiguousarray(d["dy"][:, :n])
        sub["n"] = n
        tiles.add(dig.bi_plan(dig.OP_FWD, dt, 1, k, n)[0])
        y = host(Linear(sub).forward(1), np.uint16)
        assert np.array_equal(y, y_full[:, :n]), n
    assert len(tiles) >= 3, tiles


def test_square_4096_batch_invariance_sweep():
    """W[4096,4096], X[8192,4096]: every shared row is bit-identical across
    M in {1, 3, 17, 128, 1000, 8192}; dW at M = 8192 hashed 10 times; oracle
    parity of the forward at M = 8192 on 259 sampled rows and of dW on 259
    sampled K-rows."""
    d = synth.square_4096_sweep()
    L = Linear(d)
    y = host(L.forward(1), np.uint16)
    for mp in (1, 3, 17, 128, 1000, 8192):
        assert np.array_equal(host(L.forward(1, m=mp), np.uint16), y[:mp]), mp
    rows = sample_rows(L.m, 256, 4)
    assert len(rows) >= 256
    ry = oracle.linear_forward(L.dt, d["x"], d["w"], None, L.m, L.k, L.n, rows=rows)
    check(y[rows], ry, L.dt, "square_4096_sweep fwd")
    hashes = {digest(L.dw(1)) for _ in range(10)}
    assert len(hashes) == 1
    krows = sample_rows(L.k, 256, 5)
    rw = oracle.linear_dw(L.dt, d["x"], d["dy"], L.m, L.k, L.n, rows=krows)
    check(host(L.dw(1), np.uint16)[krows], rw, L.dt, "square_4096_sweep dW")


@pytest.mark.parametrize("dt,emin,emax", [(synth.BF16, -60, 64), (synth.F16, -12, 8)],
                         ids=["bf16", "f16"])
@pytest.mark.parametrize("tc", [0, 1])
def test_output_rounding_bit_exact(dt, emin, emax, tc):
    """Reduction length 1: each output holds one exact product, so the f32
    accumulator is exact and the only rounding is the final one to the output
    type.  Operands span many binades (ties to even, overflow to inf, f16
    subnormal results), and every element of forward, dX and dW must equal the
    oracle's single round-to-nearest-even bit for bit."""
    st = np.uint16
    s = torch.cuda.current_stream()
    m, k, n = 96, 128, 192
    # forward: X[m,1] W[1,n]
    x = synth.wide_exponent_bits((m, 1), dt, 81, 0, emin, emax)
    w = synth.wide_exponent_bits((1, n), dt, 81, 1, emin, emax)
    y = empty((m, n), st)
    dig.check(dig.bi_forward(y, dev(x), dev(w), None, m, 1, n, dt, s, tc))
    ref = oracle.linear_forward(dt, x, w, None, m, 1, n)
    assert np.array_equal(host(y, st), ref.out)
    # dX = dY[m,1] W[k,1]^T
    dy = synth.wide_exponent_bits((m, 1), dt, 82, 0, emin, emax)
    wk = synth.wide_exponent_bits((k, 1), dt, 82, 1, emin, emax)
    dx = empty((m, k), st)
    dig.check(dig.bi_backward_dx(dx, dev(dy), dev(wk), m, k, 1, dt, s, tc))
    ref = oracle.linear_dx(dt, dy, wk, m, k, 1)
    assert np.array_equal(host(dx, st), ref.out)
    # dW = X[1,k]^T dY[1,n]
    x1 = synth.wide_exponent_bits((1, k), dt, 83, 0, emin, emax)
    dy1 = synth.wide_exponent_bits((1, n), dt, 83, 1, emin, emax)
    dw = empty((k, n), st)
    dig.check(dig.bi_backward_dw(dw, dev(x1), dev(dy1), 1, k, n, dt, None, 0, s, tc))
    ref = oracle.linear_dw(dt, x1, dy1, 1, k, n)
    assert np.array_equal(host(dw, st), ref.out)
    # the draws really reach overflow (and, for f16, subnormal results)
    out = host(y, st)
    assert np.any((out & 0x7FFF) == (0x7F80 if dt == synth.BF16 else 0x7C00))
    if dt == synth.F16:
        assert np.any(((out & 0x7C00) == 0) & ((out & 0x3FF) != 0))


def test_k_zero_gives_rounded_bias_and_m_zero_dw_is_zero():
    dt = synth.BF16
    b = dev(synth.normal_bits((96,), 1.0, 5, 0, dt))
    y = empty((3, 96), np.uint16)
    x = torch.empty(1, dtype=torch.int16, device="cuda")
    w = torch.empty(1, dtype=torch.int16, device="cuda")
    for tc in (0, 1):
        dig.check(dig.bi_forward(y, x, w, b, 3, 0, 96, dt, torch.cuda.current_stream(), tc))
        assert np.array_equal(host(y, np.uint16), np.tile(host(b, np.uint16), (3, 1)))
        dw = empty((70, 96), np.uint16)
        dig.check(dig.bi_backward_dw(dw, x, x, 0, 70, 96, dt, None, 0,
                                     torch.cuda.current_stream(), tc))
        assert np.all(host(dw, np.uint16) == 0)


@pytest.mark.parametrize("mkn", [(4096, 768, 3072), (2500, 96, 200)], ids=lambda s: "x".join(map(str, s)))
def test_graph_replay_matches_eager(mkn):
    """The trio captured in HIP graphs (as the benchmark replays it) gives the
    eager bytes on every replay; outputs are overwritten with garbage by eager
    work between replays.  The second shape uses the chunked dW workspace."""
    m, k, n = mkn
    d = synth.linear(m, k, n, synth.BF16, seed=31, sigma_w=0.05)
    L = Linear(d)
    ref = (digest(L.forward(1)), digest(L.dx(1)), digest(L.dw(1)))
    y, dx, dw = empty((m, n), np.uint16), empty((m, k), np.uint16), empty((k, n), np.uint16)
    nbytes = dig.bi_backward_dw_workspace_bytes(m, k, n, L.dt, 1)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        dig.check(dig.bi_forward(y, L.x, L.w, L.b, m, k, n, L.dt, cs, 1))
        dig.check(dig.bi_backward_dx(dx, L.dy, L.w, m, k, n, L.dt, cs, 1))
        dig.check(dig.bi_backward_dw(dw, L.x, L.dy, m, k, n, L.dt, ws if nbytes else None,
                                     nbytes, cs, 1))
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (y, dx, dw, ws):
            t.fill_(rep + 7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert (digest(y), digest(dx), digest(dw)) == ref, rep
