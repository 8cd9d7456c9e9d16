"""Oracle: temperature / top-k / softmax / sampling of one token per codebook.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Optimized Parler TTS", "Future work", item 2: sampling is temperature
scaling, top-k and softmax, today spread over more than ten kernels.
"Analysis and improvements": logits are produced for the last position only
(one row per codebook), the vocabulary of 1089 entries is padded to a multiple
of 8 (padding is never a candidate), and sampling runs without a GPU/CPU
synchronisation, so the random numbers are supplied as inputs (one uniform per
codebook row).

For one row x (the valid columns only), temperature T, k and uniform u:

  1. kk = min(k, V).  Rank every entry by value, largest first; equal values
     rank by the lower vocabulary index first.  The kept set S is the kk
     best-ranked indices, listed in ascending vocabulary order.
  2. T <= 0: the token is the best-ranked index (greedy).
  3. Otherwise p_i = exp((x_i - m) / T) / sum_{j in S} exp((x_j - m) / T) for
     i in S, with m the largest value (only for range; it cancels).
  4. Walk S in ascending vocabulary order accumulating p: C_r = p_{S_0} + ...
     + p_{S_r}.  The token is the first S_r with u < C_r; if rounding leaves
     u >= C_last, the token is the last element of S.

This is the inverse CDF of the top-k-filtered, temperature-scaled softmax, read
over the vocabulary in its natural order.  ``dist`` is the distance from u to
the nearest C_r: where it is tiny, either neighbour is a correct token under
rounding.
"""
import numpy as np


def kept_set(x, k):
    """(order, S): ``order`` ranks all entries (value descending, index ascending on
    ties); S = sorted(order[:min(k, len(x))])."""
    x = np.asarray(x, dtype=np.float64)
    idx = np.arange(x.shape[0])
    order = np.lexsort((idx, -x))          # last key is primary: -x, then index
    kk = min(int(k), x.shape[0])
    return order, np.sort(order[:kk])


def sample_row(x, T, k, u):
    """Returns (token, S, p, C, dist) for one row of float64 logits ``x``."""
    x = np.asarray(x, dtype=np.float64)
    order, S = kept_set(x, k)
    best = int(order[0])
    if T <= 0:
        p = (S == best).astype(np.float64)
        return best, S, p, np.cumsum(p), np.inf
    m = x[best]
    e = np.exp((x[S] - m) / float(T))
    p = e / e.sum()
    C = np.cumsum(p)
    hit = np.nonzero(float(u) < C)[0]
    r = int(hit[0]) if hit.size else len(S) - 1
    dist = float(np.min(np.abs(float(u) - C)))
    return int(S[r]), S, p, C, dist


def sample(logits, vocab_valid, T, k, u, step=None, fill_token=0):
    """Every row of ``logits`` [B, n_cb, stride] (float32 values).

    T [B], u [B, n_cb], step [B] or None.  Returns a dict with
      tokens [B, n_cb] int64        (fill_token where codebook c has not started)
      topk_idx [B, n_cb, k] int64   (S, ascending; -1 past min(k, vocab_valid))
      topk_prob [B, n_cb, k] f64    (p over S; 0 past the end)
      cdf [B, n_cb, k] f64          (C over S; 0 past the end)
      dist [B, n_cb] f64            (inf for greedy rows)
      sampled [B, n_cb] int64       (the token before the delay mask)
    """
    from .delay import apply_step_delay
    logits = np.asarray(logits)
    B, ncb, _ = logits.shape
    out = dict(tokens=np.zeros((B, ncb), np.int64),
               sampled=np.zeros((B, ncb), np.int64),
               topk_idx=np.full((B, ncb, k), -1, np.int64),
               topk_prob=np.zeros((B, ncb, k), np.float64),
               cdf=np.zeros((B, ncb, k), np.float64),
               dist=np.zeros((B, ncb), np.float64))
    for b in range(B):
        for c in range(ncb):
            x = logits[b, c, :vocab_valid].astype(np.float64)
            tok, S, p, C, dist = sample_row(x, float(T[b]), k, float(u[b, c]))
            out["sampled"][b, c] = tok
            out["topk_idx"][b, c, :len(S)] = S
            out["topk_prob"][b, c, :len(S)] = p
            out["cdf"][b, c, :len(S)] = C
            out["dist"][b, c] = dist
    out["tokens"] = apply_step_delay(out["sampled"], step, fill_token)
    return out
