"""bi_linear_backward: dX and dW of one linear layer from one call.

Where both gradients run the direct-load MFMA kernel on the 128x96 dX and
96x96 dW tiles (at least 192 dX tiles), their tiles share one launch;
elsewhere the call runs the two products in sequence.  Either way each output must carry exactly the bits of
bi_backward_dx / bi_backward_dw on the same arguments, and pass the oracle
parity rule (sampled rows of dX, sampled K-rows of dW; small-integer operands
bit-exact against the oracle)."""
import numpy as np
import pytest
import torch

import deterministic_invariant_gemm_amd as dig
import oracle
import synth
from parity import check, dev, digest, empty, host, sample_rows

pytestmark = pytest.mark.gpu

ST = {synth.F32: np.uint32, synth.BF16: np.uint16, synth.F16: np.uint16}

# shared launch: 4096x768x3072, ragged M (24 x 8 dX tiles), ragged N with K = 7 x 96
SHARED = [(4096, 768, 3072), (3001, 768, 3072), (4096, 672, 2000)]
# two launches: fewer than 192 dX tiles (M = 1000, 2048; and the narrow dX tile
# at M = 512), small shapes, chunked scalar dW, wide K
SEQUENCE = [(1000, 768, 3072), (2048, 768, 3072), (512, 768, 3072), (300, 200, 260),
            (4096, 768, 48), (1024, 2048, 512)]


def separate(d, tc=1):
    m, k, n, dt = d["m"], d["k"], d["n"], d["dt"]
    st = ST[dt]
    x, w, dy = dev(d["x"]), dev(d["w"]), dev(d["dy"])
    s = torch.cuda.current_stream()
    dx, dw = empty((m, k), st), empty((k, n), st)
    nb = dig.bi_backward_dw_workspace_bytes(m, k, n, dt, tc)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    dig.check(dig.bi_backward_dx(dx, dy, w, m, k, n, dt, s, tc), "bi_backward_dx")
    dig.check(dig.bi_backward_dw(dw, x, dy, m, k, n, dt, ws if nb else None, nb, s, tc),
              "bi_backward_dw")
    return dx, dw


def combined(d, tc=1, want_dx=True, want_dw=True):
    m, k, n, dt = d["m"], d["k"], d["n"], d["dt"]
    st = ST[dt]
    x, w, dy = dev(d["x"]), dev(d["w"]), dev(d["dy"])
    dx = empty((m, k), st) if want_dx else None
    dw = empty((k, n), st) if want_dw else None
    nb = dig.bi_backward_dw_workspace_bytes(m, k, n, dt, tc)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    ws.fill_(255)
    dig.check(dig.bi_linear_backward(dx, dw, dy, x, w, m, k, n, dt, ws if nb else None, nb,
                                     torch.cuda.current_stream(), tc), "bi_linear_backward")
    return dx, dw


@pytest.mark.parametrize("dt", [synth.BF16, synth.F16])
@pytest.mark.parametrize("shape", SHARED + SEQUENCE, ids=lambda s: "x".join(map(str, s)))
def test_same_bits_as_separate_calls(dt, shape):
    m, k, n = shape
    d = synth.linear(m, k, n, dt, seed=500 + m + k + n, sigma_w=0.05)
    print(f"linear backward dt={dt} shape={shape}", flush=True)
    dx0, dw0 = separate(d)
    dx1, dw1 = combined(d)
    assert torch.equal(dx0, dx1) and torch.equal(dw0, dw1)


@pytest.mark.parametrize("dt", [synth.BF16, synth.F16])
@pytest.mark.parametrize("shape", SHARED, ids=lambda s: "x".join(map(str, s)))
def test_shared_launch_parity_sampled(dt, shape):
    m, k, n = shape
    d = synth.linear(m, k, n, dt, seed=600 + m + k + n, sigma_w=0.05)
    print(f"linear backward parity dt={dt} shape={shape}", flush=True)
    dx, dw = combined(d)
    st = ST[dt]
    rows = sample_rows(m, 32, 11)
    rx = oracle.linear_dx(dt, d["dy"], d["w"], m, k, n, rows=rows)
    check(host(dx, st)[rows], rx, dt, f"{shape} dX")
    krows = sample_rows(k, 16, 12)
    rw = oracle.linear_dw(dt, d["x"], d["dy"], m, k, n, rows=krows)
    check(host(dw, st)[krows], rw, dt, f"{shape} dW")


def test_shared_launch_exact_integers():
    """Small-integer operands: every sum is exact in f32, so both gradients
    equal the oracle bit for bit (ragged M and N, shared launch)."""
    m, k, n = 3001, 672, 2000
    dt = synth.BF16
    d = synth.linear_integer(m, k, n, dt, seed=77, lo=-3, hi=3)
    print(f"linear backward exact integers shape={(m, k, n)}", flush=True)
    dx, dw = combined(d)
    rows = sample_rows(m, 64, 13)
    assert np.array_equal(host(dx, np.uint16)[rows],
                          oracle.linear_dx(dt, d["dy"], d["w"], m, k, n, rows=rows).out)
    krows = sample_rows(k, 48, 14)
    assert np.array_equal(host(dw, np.uint16)[krows],
                          oracle.linear_dw(dt, d["x"], d["dy"], m, k, n, rows=krows).out)


def test_one_gradient_and_determinism():
    d = synth.mlp_up_linear(synth.BF16)
    dx0, dw0 = separate(d)
    only_dx, none = combined(d, want_dw=False)
    assert none is None and torch.equal(only_dx, dx0)
    none, only_dw = combined(d, want_dx=False)
    assert none is None and torch.equal(only_dw, dw0)
    digests = {(digest(a), digest(b)) for a, b in (combined(d) for _ in range(10))}
    assert len(digests) == 1


def test_f32_and_scalar_tier():
    """f32 operands and tc = 0 run the scalar tier in two launches (same bits)."""
    for dt, tc in ((synth.F32, 1), (synth.BF16, 0)):
        d = synth.linear(257, 130, 200, dt, seed=88, sigma_w=0.05)
        dx0, dw0 = separate(d, tc)
        dx1, dw1 = combined(d, tc)
        assert torch.equal(dx0, dx1) and torch.equal(dw0, dw1), (dt, tc)


@pytest.mark.parametrize("mkn", [(4096, 768, 3072), (4096, 768, 48)],
                         ids=lambda s: "x".join(map(str, s)))
def test_graph_replay_of_the_step(mkn):
    """bi_forward + bi_linear_backward captured in a HIP graph (the shared
    launch at 4096x768x3072; two launches and the chunked dW workspace at N = 48)
    give the eager bytes on every replay, with the outputs overwritten by
    eager work between replays."""
    m, k, n = mkn
    dt = synth.BF16
    d = synth.linear(m, k, n, dt, seed=41, sigma_w=0.05)
    x, w, b, dy = dev(d["x"]), dev(d["w"]), dev(d["b"]), dev(d["dy"])
    y = empty((m, n), np.uint16)
    dig.check(dig.bi_forward(y, x, w, b, m, k, n, dt, torch.cuda.current_stream(), 1))
    dx0, dw0 = combined(d)
    ref = (digest(y), digest(dx0), digest(dw0))
    dx, dw = empty((m, k), np.uint16), empty((k, n), np.uint16)
    nb = dig.bi_backward_dw_workspace_bytes(m, k, n, dt, 1)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        dig.check(dig.bi_forward(y, x, w, b, m, k, n, dt, cs, 1))
        dig.check(dig.bi_linear_backward(dx, dw, dy, x, w, m, k, n, dt, ws if nb else None, nb,
                                         cs, 1))
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (y, dx, dw, ws):
            t.fill_(rep + 3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert (digest(y), digest(dx), digest(dw)) == ref, rep


@pytest.mark.parametrize("mkn", [(0, 96, 128), (64, 96, 0), (64, 0, 128), (1, 768, 3072)],
                         ids=lambda s: "x".join(map(str, s)))
def test_empty_and_degenerate_dims(mkn):
    """Empty reductions and empty outputs give the bytes of the two calls on
    poisoned buffers: m = 0 writes dW = +0, n = 0 writes dX = +0, k = 0 has
    no outputs; m = 1 runs the narrow dX tile and two launches."""
    m, k, n = mkn
    dt = synth.BF16
    d = synth.linear(max(m, 1), max(k, 1), max(n, 1), dt, seed=9, sigma_w=0.05)
    x, w, dy = dev(d["x"]), dev(d["w"]), dev(d["dy"])
    s = torch.cuda.current_stream()
    outs = []
    for call in ("separate", "combined"):
        dx, dw = empty((m, k), np.uint16), empty((k, n), np.uint16)
        if call == "separate":
            dig.check(dig.bi_backward_dx(dx, dy, w, m, k, n, dt, s, 1))
            dig.check(dig.bi_backward_dw(dw, x, dy, m, k, n, dt, None, 0, s, 1))
        else:
            dig.check(dig.bi_linear_backward(dx, dw, dy, x, w, m, k, n, dt, None, 0, s, 1))
        outs.append((host(dx, np.uint16), host(dw, np.uint16)))
    assert all(np.array_equal(a, b) for a, b in zip(*outs))
    if m == 0:
        assert not outs[1][1].any()
    if n == 0:
        assert not outs[1][0].any()
