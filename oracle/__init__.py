"""CPU oracle for the decode-step hot path of a Parler-TTS-style decoder.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library and imports nothing from it; the two meet
only in the seeded input generators of ``workloads``.

Every function is plain and slow on purpose: float64 NumPy, no blocking, no
fusion, no reordering beyond what the definition it follows states.

Source: the "Optimized Parler TTS" page.
  * attn.py       -- single-token self-attention over the valid prefix of a
    static causal cache, and cross-attention over the encoded description
    ("A rough architecture of Parler TTS": the description feeds
    cross-attention; "Analysis and improvements": static caches for both
    cross and causal attention, and the cost of moving the whole static cache).
  * sampling.py   -- temperature scaling, top-k, softmax and sampling of the
    next token of every codebook from supplied uniforms ("Future work", item 2;
    "Analysis and improvements": sampling without a GPU/CPU synchronisation,
    logits only for the last position, vocabulary padded to a multiple of 8).
  * delay.py      -- the delayed codebook pattern: 9 tokens per step, codebook
    c lagging c steps ("A rough architecture of Parler TTS", the delay-pattern
    figure taken from the MusicGen paper).
  * cache.py      -- writing the current token's key/value row into the
    preallocated cache ("Analysis and improvements": static caches), and the
    key order of a paged cache ("Future work": paged attention).
  * heads.py      -- the merged 9-codebook LM head on the last position and the
    merged 9-codebook embedding lookup ("Analysis and improvements").
  * rng.py        -- counter-based uniforms (Philox4x64-10 from its published
    definition), so sampling needs no random numbers from the host
    ("Analysis and improvements": sampling without a GPU/CPU synchronisation).

Every function here is pinned by a CPU test against something other than
itself (closed forms, library routines, brute force, invariants); none is
"parity unpinned".
"""
from . import attn, sampling, delay, cache, rng, heads  # noqa: F401
