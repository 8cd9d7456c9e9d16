"""Oracle: writing the current token's key and value rows into the static cache, and
reading a sequence's rows back from a paged cache.

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


def gather_paged(pool, table, block_size, layer, b, h, n):
    """Rows 0..n-1 of sequence (layer, b, h) in a paged cache, in key order: [n, hd].

    pool [NL, n_blocks, H, block_size, hd]; table [B, max_blocks] holds the physical block
    of every logical block.  Key j lives in block table[b, j // block_size] at row
    j % block_size.  The page's "Future work" names paged attention as the way to stop
    moving a whole static cache; only the rows' addresses change, not the attention.
    """
    hd = pool.shape[-1]
    out = np.empty((max(int(n), 0), hd), dtype=pool.dtype)
    for j in range(max(int(n), 0)):
        out[j] = pool[layer, table[b, j // block_size], h, j % block_size]
    return out
