"""Every tile shape of the MFMA tier -- in both kernel families (operands
staged through registers into LDS; both operands copied straight from global
memory into LDS, with the copies in bursts or spread between MFMAs) -- must give
the same bits for the same problem: the per-element MFMA sequence does not
depend on the tile.  Tiles are forced through libbi_testing.so (the same kernels
as libbi.so; its C ABI accepts tc = 16 + tile id, plus 4096 for the fp8 fast
path); ids that an op does not instantiate are rejected with BI_ERR_HIP before
any launch and skipped."""
import numpy as np
import pytest
import torch

import deterministic_invariant_gemm_amd as dig
import oracle
import synth
from parity import check, dev, empty, host

pytestmark = pytest.mark.gpu

TILE_IDS = (list(range(1, 16)) + list(range(41, 58))
            + [104, 105, 108, 111, 112, 114, 115, 116, 120, 220, 321])


def run_all(fn, ids=TILE_IDS, base=16):
    """{tile id: output bytes} for every tile the op accepts."""
    out = {}
    with dig.testing_build():
        for tid in ids:
            try:
                r = fn(base + tid)
            except dig.BIError as e:
                assert e.status == -6
                continue
            out[tid] = r
    return out


def test_production_library_rejects_forced_tiles():
    """libbi.so has no tile hook: tc = 16 + id is an unknown request there."""
    m, k, n = 64, 64, 64
    z = torch.zeros((m, n), dtype=torch.int16, device="cuda")
    s = torch.cuda.current_stream()
    assert dig.bi_forward(z, z, z, None, m, k, n, synth.BF16, s, 16 + 44) == -7
    with dig.testing_build():
        dig.check(dig.bi_forward(z, z, z, None, m, k, n, synth.BF16, s, 16 + 44))


@pytest.mark.parametrize("dt", [synth.BF16, synth.F16])
@pytest.mark.parametrize("shape", [(300, 200, 260), (520, 136, 392), (700, 264, 456),
                                   (2500, 200, 264)],
                         ids=lambda s: "x".join(map(str, s)))
def test_linear_tiles_identical(dt, shape):
    """The last shape reduces dW over three 1024-row chunks (f32 partials and
    the ordered chunk sum) in every tile."""
    m, k, n = shape
    d = synth.linear(m, k, n, dt, seed=61 + m, sigma_w=0.05)
    x, w, b, dy = dev(d["x"]), dev(d["w"]), dev(d["b"]), dev(d["dy"])
    s = torch.cuda.current_stream()

    def fwd(tc):
        y = empty((m, n), np.uint16)
        dig.check(dig.bi_forward(y, x, w, b, m, k, n, dt, s, tc))
        return host(y, np.uint16)

    def dxf(tc):
        o = empty((m, k), np.uint16)
        dig.check(dig.bi_backward_dx(o, dy, w, m, k, n, dt, s, tc))
        return host(o, np.uint16)

    def dwf(tc):
        o = empty((k, n), np.uint16)
        nb = dig.bi_backward_dw_workspace_bytes(m, k, n, dt, tc)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        dig.check(dig.bi_backward_dw(o, x, dy, m, k, n, dt, ws if nb else None, nb, s, tc))
        return host(o, np.uint16)

    refs = {"fwd": oracle.linear_forward(dt, d["x"], d["w"], d["b"], m, k, n),
            "dX": oracle.linear_dx(dt, d["dy"], d["w"], m, k, n),
            "dW": oracle.linear_dw(dt, d["x"], d["dy"], m, k, n)}
    for name, fn in (("fwd", fwd), ("dX", dxf), ("dW", dwf)):
        base = fn(1)
        check(base, refs[name], dt, f"{name} default tile")
        outs = run_all(fn)
        assert len(outs) >= 4, (name, sorted(outs))
        for tid, o in outs.items():
            assert np.array_equal(o, base), (name, tid)
        print(name, "tiles", sorted(outs))


@pytest.mark.parametrize("dt", [synth.BF16, synth.F16])
def test_grouped_tiles_identical(dt):
    d = synth.grouped(700, 136, 200, 5, dt, seed=71, pad_rows=37, empty=(3,), sigma_w=0.05)
    m, k, n, e = d["m"], d["k"], d["n"], d["e"]
    inp, wts, g = dev(d["input"]), dev(d["weights"]), dev(d["dy"])
    ids, off = dev(d["row_experts"]), dev(d["offsets"])
    s = torch.cuda.current_stream()

    def fwd(tc):
        y = empty((m, n), np.uint16)
        dig.check(dig.bi_grouped_nt(y, inp, wts, ids, off, m, k, n, e, dt, s, tc))
        return host(y, np.uint16)

    def bwd(tc):
        di = empty((m, k), np.uint16)
        dw = empty((e, n, k), np.uint32)
        dig.check(dig.bi_grouped_nt_backward(di, dw, inp, wts, g, ids, off, m, k, n, e, dt, s, tc))
        return np.concatenate([host(di, np.uint16).view(np.uint8).ravel(),
                               host(dw, np.uint32).view(np.uint8).ravel()])

    for name, fn in (("grouped fwd", fwd), ("grouped bwd", bwd)):
        base = fn(1)
        outs = run_all(fn)
        assert len(outs) >= 2, (name, sorted(outs))
        for tid, o in outs.items():
            assert np.array_equal(o, base), (name, tid)
        print(name, "tiles", sorted(outs))


FP8_TILE_IDS = [1, 4, 6, 41, 44, 46, 51, 52, 54, 55, 111, 112, 114, 115, 120, 121, 220, 321]


@pytest.mark.parametrize("shape", [(300, 256, 260), (520, 384, 392), (700, 1008, 456),
                                   (260, 200, 300)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("fast", [False, True], ids=["exact", "fast"])
def test_fp8_tiles_identical(shape, fast):
    """For either fp8 path, the register-staged fp8 kernel and every
    direct-load fp8 tile give the same bits (rows of 16-byte multiples use the
    direct-load kernel; the last shape's K = 200 sends every tile to the
    register-staged kernel)."""
    m, k, n = shape
    d = synth.fp8(m, k, n, seed=81 + m)
    a, bt = dev(d["a8"]), dev(d["bt8"])
    da = torch.tensor([float(d["da"])], dtype=torch.float32, device="cuda")
    db = torch.tensor([float(d["db"])], dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()

    def run(tc):
        y = empty((m, n), np.uint16)
        dig.check(dig.bi_fp8_mm(y, a, bt, da, db, m, k, n, s, tc))
        return host(y, np.uint16)

    base = run(dig.TC_FP8_FAST if fast else 1)
    check(base, oracle.fp8_mm(d["a8"], d["bt8"], d["da"], d["db"], m, k, n), synth.BF16,
          "fp8 default tile", groups=fast)
    outs = run_all(run, FP8_TILE_IDS, 16 + (4096 if fast else 0))
    assert len(outs) >= 3, sorted(outs)
    for tid, o in outs.items():
        assert np.array_equal(o, base), tid
    print("fp8 tiles", "fast" if fast else "exact", sorted(outs))
