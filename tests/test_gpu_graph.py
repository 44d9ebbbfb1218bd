"""The entry points only enqueue kernels on the caller's stream (no device
allocation, no memset, no host synchronisation), so a training step made of
them can be captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.  Each
replay, with eager work and host synchronisations between the replays, must
give the bytes of the same calls run eagerly: the linear step (forward, the
shared backward with a chunked dW and its workspace, the bias gradient, the
allocation-free backward), the scaled fp8 linear step (quantisers, amax
reductions, fp8 GEMMs) and the grouped GEMM with its backward."""
import numpy as np
import pytest
import torch

import deterministic_invariant_gemm_amd as dig
import synth
from parity import dev, digest, empty, f32_scalar

pytestmark = pytest.mark.gpu

REPLAYS = 3


def capture(step):
    """The step captured in a graph, after one eager run on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def replay_matches(step, outs, eager_noise):
    """Eager bytes of `outs` after `step`, then REPLAYS graph replays, each after
    the outputs were overwritten and other eager work ran, give the same bytes."""
    step()
    torch.cuda.synchronize()
    ref = [digest(t) for t in outs]
    g = capture(step)
    for r in range(REPLAYS):
        for t in outs:
            t.fill_(-1)
        eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [digest(t) for t in outs]
        assert got == ref, (r, [i for i, (a, b) in enumerate(zip(got, ref)) if a != b])


def test_linear_step_in_graph():
    # 3000 rows, K = N = 256: dW tiles are few, so dW is reduced over three
    # 1024-row chunks (f32 partials in the workspace, then the chunk sum)
    m, k, n, dt = 3000, 256, 256, synth.BF16
    d = synth.linear(m, k, n, dt, seed=131, sigma_w=0.05)
    x, w, b, dy = dev(d["x"]), dev(d["w"]), dev(d["b"]), dev(d["dy"])
    y, dx, dw = empty((m, n), np.uint16), empty((m, k), np.uint16), empty((k, n), np.uint16)
    dx2, dw2, db = empty((m, k), np.uint16), empty((k, n), np.uint16), empty((n,), np.uint16)
    nb = dig.bi_backward_dw_workspace_bytes(m, k, n, dt, 1)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    nbb = dig.bi_bias_grad_workspace_bytes(m, n, dt)
    wsb = torch.empty(max(nbb, 4), dtype=torch.uint8, device="cuda")
    other = torch.empty((64, n), dtype=torch.int16, device="cuda")

    def step():
        s = torch.cuda.current_stream()
        dig.check(dig.bi_forward(y, x, w, b, m, k, n, dt, s, 1))
        dig.check(dig.bi_linear_backward(dx, dw, dy, x, w, m, k, n, dt, ws, nb, s, 1))
        dig.check(dig.bi_bias_grad(db, dy, m, n, dt, wsb, nbb, s))
        dig.check(dig.bi_linear_backward_static(dx2, dw2, dy, x, w, m, k, n, dt, s, 1))

    def noise():
        s = torch.cuda.current_stream()
        dig.check(dig.bi_forward(other, x, w, None, 64, k, n, dt, s, 1))
        ws.fill_(7)

    replay_matches(step, [y, dx, dw, db, dx2, dw2], noise)


def test_fp8_linear_step_in_graph():
    d = synth.fp8_linear(520, 384, 392, seed=133)
    m, k, n = d["m"], d["k"], d["n"]
    x, w, g_, b = dev(d["x"]), dev(d["w"]), dev(d["g"]), dev(d["b"])
    sc = {key: f32_scalar(float(d[key])) for key in
          ("sx", "sw", "sg", "sx_inv", "sw_inv", "sg_inv")}
    nb = dig.bi_fp8_linear_workspace_bytes(m, k, n)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    amax = torch.zeros(3, dtype=torch.float32, device="cuda")
    y, dx, dw = empty((m, n), np.uint16), empty((m, k), np.uint16), empty((n, k), np.uint16)

    def step():
        s = torch.cuda.current_stream()
        dig.check(dig.bi_fp8_linear_forward(y, x, w, b, sc["sx"], sc["sw"], sc["sx_inv"],
                                            sc["sw_inv"], amax[0:1], amax[1:2], m, k, n, ws, nb,
                                            s, 1))
        dig.check(dig.bi_fp8_linear_backward(dx, dw, g_, x, w, sc["sg"], sc["sw"], sc["sx"],
                                             sc["sg_inv"], sc["sw_inv"], sc["sx_inv"],
                                             amax[2:3], m, k, n, ws, nb, s, 1))

    def noise():
        ws.fill_(3)
        amax.fill_(-5.0)

    replay_matches(step, [y, dx, dw, amax], noise)


@pytest.mark.parametrize("case", [
    (700, 136, 200, 5, 37, (3,), 135),
    # the forward's 256x256 grid holds more than one round: the split launch
    # (whole tiles, then 256x128 halves chosen on the device from the offsets)
    (16384, 256, 1408, 8, 819, (), 5),
], ids=["small", "split"])
def test_grouped_step_in_graph(case):
    m, k, n, e, pad, empty_x, seed = case
    d = synth.grouped(m, k, n, e, synth.BF16, seed=seed, pad_rows=pad, empty=empty_x,
                      sigma_w=0.05)
    inp, wts, gy = dev(d["input"]), dev(d["weights"]), dev(d["dy"])
    ids, off = dev(d["row_experts"]), dev(d["offsets"])
    y, di = empty((m, n), np.uint16), empty((m, k), np.uint16)
    dwt = empty((e, n, k), np.uint32)

    def step():
        s = torch.cuda.current_stream()
        dig.check(dig.bi_grouped_nt(y, inp, wts, ids, off, m, k, n, e, synth.BF16, s, 1))
        dig.check(dig.bi_grouped_nt_backward(di, dwt, inp, wts, gy, ids, off, m, k, n, e,
                                             synth.BF16, s, 1))

    def noise():
        pass

    replay_matches(step, [y, di, dwt], noise)
