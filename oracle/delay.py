"""Oracle: the delayed codebook pattern.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Optimized Parler TTS", "A rough architecture of Parler TTS": at every step
the decoder emits one token for each of the 9 DAC codebooks in parallel,
following a delayed pattern (the figure there comes from the MusicGen paper).
Reading: codebook c (0-based) lags codebook 0 by c steps, so at decode step s
(the number of steps already taken, 0 for the first generated step) codebook
c has started iff s >= c; before that it emits a fill token.  Audio frame f's
codebook-c token is therefore produced at step f + c.
"""
import numpy as np


def codebook_started(step, c):
    """True where codebook ``c`` emits a real token at decode step ``step``."""
    return np.asarray(step) >= c


def apply_step_delay(sampled, step, fill_token):
    """tokens[b, c] = sampled[b, c] if step[b] >= c else fill_token (step None: no mask)."""
    sampled = np.asarray(sampled)
    if step is None:
        return sampled.copy()
    B, ncb = sampled.shape
    out = sampled.copy()
    for b in range(B):
        for c in range(ncb):
            if not codebook_started(step[b], c):
                out[b, c] = fill_token
    return out


def delay_frames(frames, fill_token):
    """Frames [F, n_cb] -> the delayed step matrix [F + n_cb - 1, n_cb]:
    out[s, c] = frames[s - c, c] when 0 <= s - c < F, else fill_token."""
    frames = np.asarray(frames)
    F, ncb = frames.shape
    out = np.full((F + ncb - 1, ncb), fill_token, dtype=frames.dtype)
    for s in range(F + ncb - 1):
        for c in range(ncb):
            if 0 <= s - c < F:
                out[s, c] = frames[s - c, c]
    return out


def undelay(steps):
    """Step matrix [S, n_cb] -> the S - n_cb + 1 complete frames [F, n_cb]:
    frame f's codebook-c token is steps[f + c, c]."""
    steps = np.asarray(steps)
    S, ncb = steps.shape
    F = S - ncb + 1
    out = np.empty((max(F, 0), ncb), dtype=steps.dtype)
    for f in range(F):
        for c in range(ncb):
            out[f, c] = steps[f + c, c]
    return out
