"""Oracle: the merged 9-codebook LM head on the last position, and the merged
9-codebook embedding lookup.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Optimized Parler TTS", "Analysis and improvements":
  * logits are computed for the last position only, and the nine per-codebook LM
    heads are merged into one weight matrix, so one matrix-vector product per
    sequence produces all nine rows of logits;
  * the nine embedding lookups (one per codebook) are merged into one gather.
"A rough architecture of Parler TTS": the decoder consumes the nine tokens of the
previous step at once (MusicGen-style), so its input is the sum of the nine
codebooks' embedding rows.

  lm_head:  logits[b, c, v] = sum_d h[b, d] * W[c, v, d]    for v < V_valid
            (no bias; columns v >= V_valid of the output are not part of the result)
  embed:    x[b, d] = sum_c E[c, tokens[b, c], d]            tokens outside
            [0, V_emb) contribute nothing
Values are taken exactly (bf16 bit patterns decoded to float64) and summed in float64.
"""
import numpy as np

from .attn import bf16_bits_to_f64


def _f64(x):
    x = np.asarray(x)
    return bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def lm_head(h, W, V_valid):
    """h [B, D], W [n_cb, V_stride, D] -> logits [B, n_cb, V_valid] float64."""
    hf, Wf = _f64(h), _f64(W)
    n_cb = Wf.shape[0]
    out = np.empty((hf.shape[0], n_cb, V_valid), np.float64)
    for c in range(n_cb):
        out[:, c, :] = hf @ Wf[c, :V_valid, :].T
    return out


def embed(tokens, E):
    """tokens [B, n_cb] int, E [n_cb, V_emb, D] -> x [B, D] float64."""
    Ef = _f64(E)
    n_cb, V_emb, D = Ef.shape
    tokens = np.asarray(tokens)
    x = np.zeros((tokens.shape[0], D), np.float64)
    for b in range(tokens.shape[0]):
        for c in range(n_cb):
            t = int(tokens[b, c])
            if 0 <= t < V_emb:
                x[b] += Ef[c, t]
    return x
