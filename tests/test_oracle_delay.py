"""Pins for the delay-pattern oracle (CPU only)."""
import os

import numpy as np

from oracle import delay as D
from workloads import configs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "delay_pattern_4frames_9codebooks.txt")


def _read_golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([-1 if t == "-" else int(t) for t in line.split()])
    return np.array(rows)


def test_golden_delay_pattern():
    frames = np.tile(np.arange(4).reshape(4, 1), (1, 9))      # frame index as the token
    got = D.delay_frames(frames, -1)
    assert np.array_equal(got, _read_golden())


def test_codebook_c_first_emits_at_step_c():
    ncb = configs.N_CODEBOOKS
    steps = np.arange(30)
    sampled = np.full((30, ncb), 7)
    toks = D.apply_step_delay(sampled, steps, -1)
    for c in range(ncb):
        first = int(np.nonzero(toks[:, c] != -1)[0][0])
        assert first == c
        assert np.all(toks[:c, c] == -1) and np.all(toks[c:, c] == 7)


def test_delay_undelay_round_trip():
    rng = np.random.default_rng(0)
    for F in (1, 2, 17):
        frames = rng.integers(0, 1089, size=(F, 9))
        d = D.delay_frames(frames, 1089)
        assert d.shape == (F + 8, 9)
        assert np.array_equal(D.undelay(d), frames)
        assert np.array_equal(D.delay_frames(D.undelay(d), 1089), d)


def test_no_step_means_no_mask():
    s = np.arange(18).reshape(2, 9)
    assert np.array_equal(D.apply_step_delay(s, None, -1), s)


def test_vocabulary_padding_is_the_next_multiple_of_eight():
    assert configs.VOCAB_PADDED % 8 == 0
    assert 0 <= configs.VOCAB_PADDED - configs.VOCAB_VALID < 8
