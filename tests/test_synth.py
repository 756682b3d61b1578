"""The seeded input generators (CPU): the counter-based weight hash gives the same fp32 bits
from numpy and from torch, for any block of rows and columns drawn on its own, so a weight too
large for the host can be drawn on the device while the oracle draws only the parts it checks."""
import numpy as np
import torch

import synth


def test_hash_weight_numpy_matches_torch():
    for row0, nrows, cols, seed in ((0, 8, 64, 0), (5, 3, 4096, 11), ((1 << 20) - 4, 4, 4096, 11),
                                    ((1 << 22) - 2, 2, 1024, 7)):
        a = synth.hash_weight(np.arange(row0, row0 + nrows), np.arange(cols), seed)
        b = synth.hash_weight_rows_torch(row0, nrows, cols, seed, "cpu").numpy()
        assert a.dtype == np.float32 and b.dtype == np.float32
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (row0, nrows, cols, seed)


def test_hash_weight_blocks_are_consistent():
    """A column block drawn alone equals the same columns of the full rows."""
    full = synth.hash_weight(np.arange(100, 110), np.arange(4096), 3)
    block = synth.hash_weight(np.arange(100, 110), np.arange(2368, 2432), 3)
    assert np.array_equal(full[:, 2368:2432].view(np.uint32), block.view(np.uint32))


def test_hash_weight_range_and_spread():
    w = synth.hash_weight(np.arange(256), np.arange(1024), 11).astype(np.float64)
    assert w.min() >= -2.0 ** -5 and w.max() < 2.0 ** -5
    # uniform on [-2^-5, 2^-5): mean ~0, standard deviation 2^-5 / sqrt(3)
    assert abs(w.mean()) < 2e-4
    assert abs(w.std() - 2.0 ** -5 / np.sqrt(3)) < 2e-4
    # every value is a multiple of 2^-28 (exact in fp32)
    assert np.all(np.mod(w * 2.0 ** 28, 1.0) == 0)
