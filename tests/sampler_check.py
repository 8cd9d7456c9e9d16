"""The sampler's parity bars against the oracle, shared by the GPU sampler tests.

* Top-k index sets: bit-exact, padded with -1 (probabilities 0) past min(k, V).
* Probabilities: the kernels form the weights exp((x - m) / T) and their sum in float64
  and round each probability once to float32, so each is within half an ulp of the
  oracle's: |p - p*| <= 2^-24 p* (with float64 slack).  Greedy rows (T <= 0) are one-hot.
* CDF: the kernels compare the uniform with the float64 running sum of the exported
  probabilities in vocabulary order, so the running sum of what they export IS the CDF
  they sample from.  Its error against the oracle's is at most the sum of the roundings,
  |C_r - C*_r| <= 2^-24 C*_r (plus float64 summation), about 6e-8: well inside the 5e-7
  bar that the GPU CDF must meet, which is itself held too.
* Tokens: exact, except rows whose uniform lies within 1e-6 of an oracle CDF boundary
  (either neighbour is then correct under rounding).  With the CDF error above, a
  mismatch can only occur within 1e-7 of a boundary, which is also asserted, and the
  excluded rows must be few: at most max(2, rows / 1000) (expected about 1e-4 per row
  at k = 50).
"""
import numpy as np

BAND = 1e-6          # token exclusion band around an oracle CDF boundary
CDF_BAR = 5e-7       # the GPU CDF accuracy bar
ULP = 2.0 ** -24     # half an ulp of float32, relative


def check(want, tokens, idx, prob, T, k, V, fill_rows_ok=True):
    """Compares one sampler call with the oracle's result ``want``; returns stats."""
    kk = min(k, V)
    assert np.array_equal(idx[..., :kk], want["topk_idx"][..., :kk]), "top-k sets differ"
    assert np.all(idx[..., kk:] == -1) and np.all(prob[..., kk:] == 0)
    n_cb = tokens.shape[1]
    sampling = np.asarray(T, np.float64)[:, None].repeat(n_cb, 1) > 0
    p_g = prob[..., :kk].astype(np.float64)
    p_w = want["topk_prob"][..., :kk]
    # greedy rows: one-hot, exactly
    assert np.array_equal(p_g[~sampling], p_w[~sampling])
    perr = cerr = 0.0
    if sampling.any():
        pg, pw = p_g[sampling], p_w[sampling]
        pbar = np.maximum(pw * ULP, 2.0 ** -150) * (1 + 1e-6)
        assert np.all(np.abs(pg - pw) <= pbar), float(np.max(np.abs(pg - pw) / np.maximum(pw, 1e-300)))
        perr = float(np.max(np.abs(pg - pw)))
        cg = np.cumsum(pg, axis=-1)
        cw = want["cdf"][..., :kk][sampling]
        cbar = cw * ULP * (1 + 1e-6) + kk * 2.0 ** -52
        assert np.all(np.abs(cg - cw) <= cbar), float(np.max(np.abs(cg - cw)))
        cerr = float(np.max(np.abs(cg - cw)))
        assert cerr <= CDF_BAR
    near = want["dist"] < BAND
    mismatch = tokens != want["tokens"]
    assert not (mismatch & ~near).any(), f"token mismatch at {np.argwhere(mismatch & ~near)[:5]}"
    assert not (mismatch & (want["dist"] >= 1e-7)).any(), "mismatch farther than the CDF error"
    excluded = int(near.sum())
    assert excluded <= max(2, tokens.size // 1000), excluded
    return dict(rows=int(tokens.size), excluded=excluded, prob_err=perr, cdf_err=cerr,
                mismatched=int(mismatch.sum()))
