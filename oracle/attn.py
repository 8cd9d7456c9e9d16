"""Oracle: single-query softmax attention over the valid prefix of a static cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Optimized Parler TTS", "Analysis and improvements": the decoder keeps static,
preallocated caches for both the causal self-attention and the cross-attention
over the description, so every tensor keeps one address; the drawback named
there is that attention then moves the whole cache each step.  What the step
must compute is unchanged by where the cache lives: for the one new token,
softmax attention over the keys and values that are actually valid.  For a
single query, "causal" means every slot up to and including the current token,
i.e. the first ``len[b]`` slots of the sequence (the current token's key and
value are already in the cache).  "A rough architecture of Parler TTS": the
description, encoded once, is what cross-attention attends to; the same
function serves it with the description length in place of ``len``.

The result is the plain definition, in float64 from the exact input values:

    n     = min(len, capacity)            (n <= 0: the output is all zeros)
    s_j   = scale * sum_d q_d K_jd        for j < n
    w_j   = exp(s_j - max_j s_j)
    o_d   = sum_j w_j V_jd / sum_j w_j

Subtracting the maximum changes nothing mathematically; it only keeps exp in
range.
"""
import numpy as np


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64 values, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _to_f64(x, dtype):
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def attend_one(q, K, V, n, scale):
    """Attention of one query ``q`` [hd] over the first ``n`` rows of ``K``, ``V`` [L, hd].

    All arguments are float64 values (rows beyond ``n`` are never touched).
    """
    hd = q.shape[-1]
    n = min(int(n), K.shape[0])
    if n <= 0:
        return np.zeros(hd, dtype=np.float64)
    s = scale * (K[:n] @ q)
    w = np.exp(s - s.max())
    return (w @ V[:n]) / w.sum()


def attention_rows(q, K, V, lens, scale, dtype, rows):
    """Oracle output for selected (layer, b, h) rows only.

    q [NL,B,H,hd], K and V [NL,B,H,cap,hd] in the input dtype ("bf16" bit patterns
    or "f32"), lens [B]; rows is a list of (layer, b, h).  Returns [len(rows), hd]
    float64.  Only the valid prefix of each selected row is decoded.
    """
    cap = K.shape[3]
    out = np.zeros((len(rows), q.shape[-1]), dtype=np.float64)
    for r, (layer, b, h) in enumerate(rows):
        n = min(int(lens[b]), cap)
        if n <= 0:
            continue
        out[r] = attend_one(_to_f64(q[layer, b, h], dtype),
                            _to_f64(K[layer, b, h, :n], dtype),
                            _to_f64(V[layer, b, h, :n], dtype), n, scale)
    return out


def attention(q, K, V, lens, scale, dtype):
    """Oracle output for every (layer, b, h): [NL, B, H, hd] float64."""
    NL, B, H, hd = q.shape
    rows = [(layer, b, h) for layer in range(NL) for b in range(B) for h in range(H)]
    return attention_rows(q, K, V, lens, scale, dtype, rows).reshape(NL, B, H, hd)


def attend_masked(q, K, V, n, mask, scale):
    """Attention of ``q`` over the keys j < n with ``mask[j]`` true (a boolean mask
    over the description; "A rough architecture of Parler TTS": cross-attention reads
    the encoded description, whose padding an attention mask hides).  No key
    attended: zeros.  All arguments are float64 values except the boolean mask."""
    hd = q.shape[-1]
    n = min(int(n), K.shape[0])
    keep = np.nonzero(np.asarray(mask[:max(n, 0)], dtype=bool))[0]
    if keep.size == 0:
        return np.zeros(hd, dtype=np.float64)
    s = scale * (K[keep] @ q)
    w = np.exp(s - s.max())
    return (w @ V[keep]) / w.sum()


def round_bf16(x):
    """float32 values rounded to bfloat16 (nearest, ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)) << np.uint32(16)
    return r.astype(np.uint32).view(np.float32)
