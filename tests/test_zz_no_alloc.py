"""bi_linear_backward_static: the allocation-free variant of
bi_linear_backward (dW's f32 chunk partials in the library's static per-GPU
array) gives the bytes of bi_linear_backward with a caller workspace, on two
calls in a row with the second smaller (the array keeps the first call's
partials, which the second must overwrite, not read), on the MFMA and scalar
tiers; beyond the array's size it refuses before enqueuing anything."""
import numpy as np
import pytest
import torch

import deterministic_invariant_gemm_amd as dig
import synth
from parity import dev, digest, empty

pytestmark = pytest.mark.gpu

ST = {synth.F32: np.uint32, synth.BF16: np.uint16, synth.F16: np.uint16}


def both(d, tc):
    """(workspace call's dx, dw), (static call's dx, dw) on the same inputs."""
    m, k, n, dt = d["m"], d["k"], d["n"], d["dt"]
    st = ST[dt]
    x, w, dy = dev(d["x"]), dev(d["w"]), dev(d["dy"])
    s = torch.cuda.current_stream()
    nb = dig.bi_backward_dw_workspace_bytes(m, k, n, dt, tc)
    assert 0 < nb <= dig.BI_STATIC_SCRATCH_BYTES, nb  # chunked dW: the scratch is used
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ref = (empty((m, k), st), empty((k, n), st))
    dig.check(dig.bi_linear_backward(ref[0], ref[1], dy, x, w, m, k, n, dt, ws, nb, s, tc))
    out = (empty((m, k), st), empty((k, n), st))
    dig.check(dig.bi_linear_backward_static(out[0], out[1], dy, x, w, m, k, n, dt, s, tc))
    return ref, out


@pytest.mark.parametrize("dt,tc", [(synth.BF16, 1), (synth.F16, 1), (synth.F32, 1),
                                   (synth.BF16, 0)], ids=["bf16", "f16", "f32", "bf16-scalar"])
def test_static_backward_matches_workspace_call(dt, tc):
    # first call: 8 chunks of 1024 rows (MFMA) / 20 of 256 (scalar); second:
    # a smaller problem with fewer chunks, over the first call's partials
    shapes = [(8192, 256, 512), (2500, 200, 264)] if tc else [(5120, 128, 128), (700, 96, 72)]
    for i, (m, k, n) in enumerate(shapes):
        print(f"static backward dt={dt} tc={tc} call {i}: {m}x{k}x{n}", flush=True)
        d = synth.linear(m, k, n, dt, seed=90 + i, sigma_w=0.05)
        ref, out = both(d, tc)
        assert digest(out[0]) == digest(ref[0]), ("dX", i)
        assert digest(out[1]) == digest(ref[1]), ("dW", i)


def test_static_backward_one_gradient_and_limit():
    d = synth.linear(4096, 256, 384, synth.BF16, seed=97, sigma_w=0.05)
    m, k, n = d["m"], d["k"], d["n"]
    x, w, dy = dev(d["x"]), dev(d["w"]), dev(d["dy"])
    s = torch.cuda.current_stream()
    nb = dig.bi_backward_dw_workspace_bytes(m, k, n, synth.BF16, 1)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ref = empty((k, n), np.uint16)
    dig.check(dig.bi_backward_dw(ref, x, dy, m, k, n, synth.BF16, ws, nb, s, 1))
    only_dw = empty((k, n), np.uint16)
    dig.check(dig.bi_linear_backward_static(None, only_dw, dy, x, w, m, k, n, synth.BF16, s, 1))
    assert digest(only_dw) == digest(ref)
    # partials of 64 chunks of [1024, 1024] f32 (256 MiB) exceed the array: refused,
    # nothing enqueued (the output keeps its poison)
    big_m, big_k, big_n = 65536, 1024, 1024
    assert dig.bi_backward_dw_workspace_bytes(big_m, big_k, big_n, synth.BF16, 1) > \
        dig.BI_STATIC_SCRATCH_BYTES
    poison = digest(only_dw)
    assert dig.bi_linear_backward_static(None, only_dw, dy, x, w, big_m, big_k, big_n,
                                         synth.BF16, s, 1) == -5
    assert digest(only_dw) == poison
