"""Oracle: counter-based uniforms for sampling without host input.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Optimized Parler TTS", "Analysis and improvements": the decode step samples
without a GPU/CPU synchronisation.  With the random numbers generated on the
device from a counter, a captured step needs no host input at all.  The
generator is Philox4x64 with 10 rounds, as published by Salmon, Moraes, Dror
and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011): a counter
of four 64-bit words and a key of two 64-bit words go through ten rounds of

  (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0,  lo(M1 c2),
                       hi(M0 c0) ^ c3 ^ k1,  lo(M0 c0))

where hi/lo are the upper and lower 64 bits of the 128-bit product, with the
key bumped by the Weyl constants (W0, W1) between rounds.

Uniform for row (b, c) at step s: counter (s, b, c, 0), key (seed, 0); the
top 24 bits of output word 0 scaled by 2^-24, a value in [0, 1) that float32
holds exactly.
"""
import numpy as np

M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
MASK64 = (1 << 64) - 1


def philox4x64_10(counter, key):
    """The four output words for a counter (4 ints) and key (2 ints), as Python ints."""
    c = [int(x) & MASK64 for x in counter]
    k = [int(x) & MASK64 for x in key]
    for r in range(10):
        p0 = M0 * c[0]
        p1 = M1 * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k[0], p1 & MASK64, (p0 >> 64) ^ c[3] ^ k[1], p0 & MASK64]
        if r < 9:
            k = [(k[0] + W0) & MASK64, (k[1] + W1) & MASK64]
    return c


def uniform_from_word(w):
    """[0, 1) from the top 24 bits of a 64-bit word (exact in float32)."""
    return np.float32((int(w) >> 40) * 2.0 ** -24)


def sample_uniforms(seed, steps, n_cb):
    """[B, n_cb] float32 uniforms for a step: steps[b] is the step of sequence b
    (None: step 0 for every sequence)."""
    B = len(steps) if steps is not None else 1
    u = np.zeros((B, n_cb), np.float32)
    for b in range(B):
        s = int(steps[b]) if steps is not None else 0
        for c in range(n_cb):
            u[b, c] = uniform_from_word(philox4x64_10((s & MASK64, b, c, 0), (seed, 0))[0])
    return u
