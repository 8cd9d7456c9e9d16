"""Pins for oracle/rng.py (counter-based uniforms), CPU only.

The generator is pinned against NumPy's own Philox bit generator, an
independent implementation of the same published Philox4x64-10 block function.
NumPy's generator advances its 256-bit counter by one before producing each
block, so the block for counter X is its first output after seeding with X - 1.
"""
import numpy as np
import pytest

from oracle import rng

MASK = (1 << 64) - 1


def numpy_block(counter, key):
    """Philox4x64-10 output for `counter` via NumPy (counter - 1 as a 256-bit integer)."""
    v = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    v = (v - 1) % (1 << 256)
    c = np.array([(v >> (64 * i)) & MASK for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=c, key=np.array([int(k) for k in key], dtype=np.uint64))
    return [int(x) for x in bg.random_raw(4)]


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4, 5, 6, 7])
def test_block_matches_numpy_philox(seed):
    r = np.random.default_rng(seed)
    ctr = [int(x) for x in r.integers(0, 2**64, 4, dtype=np.uint64)]
    key = [int(x) for x in r.integers(0, 2**64, 2, dtype=np.uint64)]
    assert rng.philox4x64_10(ctr, key) == numpy_block(ctr, key)


@pytest.mark.parametrize("ctr,key", [
    ((0, 0, 0, 0), (0, 0)),                       # counter 0: NumPy wraps from 2^256 - 1
    ((0, 5, 0, 0), (123, 0)),                     # borrow out of word 0
    ((MASK, MASK, MASK, MASK), (MASK, MASK)),     # all ones
    ((7, 0, 3, 0), (20261202, 0)),                # the layout the sampler uses
])
def test_block_edge_counters_match_numpy(ctr, key):
    assert rng.philox4x64_10(ctr, key) == numpy_block(ctr, key)


def test_uniform_mapping_edges():
    assert rng.uniform_from_word(0) == np.float32(0.0)
    top = rng.uniform_from_word(MASK)
    assert top == np.float32(1.0 - 2.0 ** -24) and top < 1.0
    assert rng.uniform_from_word(1 << 40) == np.float32(2.0 ** -24)
    assert rng.uniform_from_word((1 << 40) - 1) == np.float32(0.0)   # only the top 24 bits count


def test_uniforms_layout_and_statistics():
    seed = 99
    steps = np.arange(64)
    u = rng.sample_uniforms(seed, steps, 9)
    assert u.shape == (64, 9) and u.dtype == np.float32
    # each entry is the first word of its own block: counter (step, b, c, 0), key (seed, 0)
    for b, c in [(0, 0), (5, 3), (63, 8)]:
        w = rng.philox4x64_10((int(steps[b]), b, c, 0), (seed, 0))[0]
        assert u[b, c] == np.float32((w >> 40) * 2.0 ** -24)
    assert np.all((u >= 0) & (u < 1))
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))       # on the 2^-24 grid
    flat = u.ravel()
    assert abs(flat.mean() - 0.5) < 4 * (1 / np.sqrt(12)) / np.sqrt(flat.size)
    hist = np.histogram(flat, bins=8, range=(0, 1))[0]
    exp = flat.size / 8
    assert np.all(np.abs(hist - exp) < 5 * np.sqrt(exp))
    assert len(np.unique(flat)) > 0.99 * flat.size


def test_no_step_means_step_zero_and_seed_changes_everything():
    a = rng.sample_uniforms(5, None, 9)
    b = rng.sample_uniforms(5, [0], 9)
    c = rng.sample_uniforms(6, [0], 9)
    assert np.array_equal(a, b)
    assert not np.any(a == c)
