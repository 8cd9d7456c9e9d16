"""Oracle: writing the current token's key and value rows into the static cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Optimized Parler TTS", "Analysis and improvements": the self-attention caches
are preallocated at a fixed capacity, so every step writes the new token's key
and value into the next row instead of growing a tensor.  Here len[b] already
counts the current token, so its row is len[b] - 1; lengths outside
[1, L_cap] write nothing.
"""
import numpy as np


def append(k_new, v_new, k_cache, v_cache, lens):
    """k_new, v_new [NL, B, H, hd]; caches [NL, B, H, L_cap, hd] (modified in place)."""
    L_cap = k_cache.shape[3]
    for b, n in enumerate(lens):
        n = int(n)
        if 1 <= n <= L_cap:
            k_cache[:, b, :, n - 1, :] = k_new[:, b, :, :]
            v_cache[:, b, :, n - 1, :] = v_new[:, b, :, :]
    return k_cache, v_cache
