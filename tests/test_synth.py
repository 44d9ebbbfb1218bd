"""Host checks of the input generators: the closed-form integer generator gives
the same values from numpy and from torch, for any block of a large index
space, within its range, and different rows differ."""
import numpy as np
import torch

import synth


def test_hashed_ints_backends_agree_and_blocks_compose():
    rows, cols = np.array([0, 1, 7, 466034, 2**31 + 5]), np.arange(40)
    a = synth.hashed_ints(rows, cols, -4, 3, 91, 0)
    b = synth.hashed_ints(torch.from_numpy(rows), torch.from_numpy(cols), -4, 3, 91, 0,
                          xp=torch).numpy()
    assert np.array_equal(a, b)
    assert a.min() >= -4 and a.max() <= 3 and set(np.unique(a)) == set(range(-4, 4))
    # a block equals the same block cut from a larger one
    full = synth.hashed_ints(np.arange(64), np.arange(64), -1, 1, 5, 2)
    part = synth.hashed_ints(np.arange(10, 20), np.arange(30, 50), -1, 1, 5, 2)
    assert np.array_equal(full[10:20, 30:50], part)
    # rows are distinct (an index off by any amount reads different values)
    many = synth.hashed_ints(np.arange(4096), np.arange(64), -4, 3, 91, 0)
    assert len({r.tobytes() for r in many}) == 4096
