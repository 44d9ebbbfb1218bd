"""GPU parity of the bias gradient (column sums of dY, f32 accumulation, one
rounding) against the oracle: several 256-row chunks with ragged tails, the
element load path (odd n, misaligned dY) against the vector path, m = 0,
9000 x 72 (35 chunks: the chunk sum's 16-wide loads and its tail), the full
4096 x 3072 bf16 shape, and run-to-run equality."""
import numpy as np
import pytest
import torch

import deterministic_invariant_gemm_amd as dig
import oracle
import synth
from parity import check, dev, digest, empty, host

pytestmark = pytest.mark.gpu

ST = {synth.F32: np.uint32, synth.BF16: np.uint16, synth.F16: np.uint16}


def bias_grad(dy, m, n, dt):
    db = empty((n,), ST[dt])
    nbytes = dig.bi_bias_grad_workspace_bytes(m, n, dt)
    ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device="cuda")
    ws.fill_(255)
    dig.check(dig.bi_bias_grad(db, dy, m, n, dt, ws if nbytes else None, nbytes,
                               torch.cuda.current_stream()), "bi_bias_grad")
    return db


@pytest.mark.parametrize("dt", [synth.F32, synth.BF16, synth.F16])
@pytest.mark.parametrize("m,n", [(1, 8), (256, 256), (257, 264), (1000, 520), (517, 77),
                                 (3, 1), (2049, 24), (9000, 72)])
def test_bias_grad_parity(dt, m, n):
    dy = synth.normal_bits((m, n), 1.0, 31, 5, dt)
    print(f"bias_grad dt={dt} m={m} n={n}", flush=True)
    got = host(bias_grad(dev(dy), m, n, dt), ST[dt])
    check(got, oracle.bias_grad(dt, dy, m, n), dt, f"db {dt} {m}x{n}")


@pytest.mark.parametrize("dt", [synth.BF16, synth.F32])
def test_element_path_matches_vector_path(dt):
    m, n = 700, 512
    dy = synth.normal_bits((m, n), 1.0, 32, 5, dt)
    d = dev(dy)
    vec = digest(bias_grad(d, m, n, dt))
    # the same values at an address that is not 16-byte aligned
    esz = 4 if dt == synth.F32 else 2
    flat = dev(np.concatenate([np.zeros(1, ST[dt]), dy.reshape(-1)]))
    shifted = flat.data_ptr() + esz
    assert shifted % 16 != 0
    elem = digest(bias_grad(shifted, m, n, dt))
    assert vec == elem


def test_empty_batch_writes_zero():
    db = bias_grad(None, 0, 100, synth.BF16)
    assert np.all(host(db, np.uint16) == 0)


def test_full_shape_parity_and_determinism():
    m, n, dt = 4096, 3072, synth.BF16
    dy = synth.normal_bits((m, n), 1.0, 2, 4, dt)
    d = dev(dy)
    got = bias_grad(d, m, n, dt)
    h = digest(got)
    for _ in range(3):
        assert digest(bias_grad(d, m, n, dt)) == h
    check(host(got, np.uint16), oracle.bias_grad(dt, dy, m, n), dt, "db 4096x3072")
