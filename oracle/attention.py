"""Materialised three-pass softmax attention in float64 (oracle; test infrastructure).

Definition followed -- the "GPU优化" tag page (guijiagi.com), excerpt "Flash Attention解决了
什么问题？", part 算法原理 / 标准注意力计算: the score matrix is Q times K-transposed divided by
the square root of the head dimension, P is its row-wise softmax and the output is P times V.
Here the divisor is an explicit ``scale`` argument (the workloads pass 1/sqrt(d)).

The softmax is done the way "FlashAttention优化" (coreui.cn) §2.2 describes the standard,
unfused implementation: a first pass for the row maximum, a second pass for the exponentials
and their sum, a third pass that normalises.  The whole N x N matrix is materialised; that is
exactly what the fused GPU kernel avoids, and why this is slow but easy to check by eye.

Readings of points the pages leave open:
* log-sum-exp stored per row is the natural-log LSE of the *scaled* scores,
  ``m + ln(l)`` (page "Gemini 3 Flash的注意力内核重写" §4 keeps a row maximum and a
  normaliser for the backward pass; the two are folded into one number).
* causal: square N x N, key j is visible to query i iff j <= i.
* padding: with per-sequence lengths L_b, keys j >= L_b are invisible; query rows i >= L_b
  are padding and get O = 0, LSE = -inf.
* grouped-query heads: query head h reads kv head h // (H // Hkv) (consecutive groups).
"""

import numpy as np

__all__ = ["attention_ref", "attention_probs_ref"]


def _visible_keys(rows, L, causal):
    """Number of visible keys for each query row (keys 0..count-1 are visible)."""
    rows = np.asarray(rows, dtype=np.int64)
    if causal:
        return np.minimum(rows + 1, L)
    return np.full(rows.shape, L, dtype=np.int64)


def _three_pass(q_rows, k, v, scale, counts):
    """Three-pass softmax attention for a set of query rows against one key/value sequence.

    q_rows [n, d], k [L, d], v [L, d] float64; counts[i] = visible keys of row i (>= 1).
    Returns O [n, d], LSE [n], P [n, L].
    """
    L = k.shape[0]
    # pass 1: scaled scores, mask, row maximum
    s = scale * (q_rows @ k.T)
    invisible = np.arange(L)[None, :] >= counts[:, None]
    s = np.where(invisible, -np.inf, s)
    m = s.max(axis=1)
    # pass 2: exponentials relative to the maximum and their row sums
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    # pass 3: normalise, weight the values, log-sum-exp
    p = e / l[:, None]
    o = p @ v
    lse = m + np.log(l)
    return o, lse, p


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d] / [B, Hkv, N, d]")
    B, H, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if k.shape != v.shape or Bk != B or Nk != N or dk != d:
        raise ValueError("k and v must be [B, Hkv, N, d] matching q")
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    return B, H, Hkv, N, d


def _lengths(seq_lens, B, N):
    if seq_lens is None:
        return [N] * B
    lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    if len(lens) != B or any(x < 0 or x > N for x in lens):
        raise ValueError("seq_lens must hold B values in [0, N]")
    return lens


def attention_ref(q, k, v, scale, causal=False, seq_lens=None, rows=None):
    """Attention forward, materialised, fp64.

    q [B, H, N, d]; k, v [B, Hkv, N, d] (any real dtype; upcast exactly to float64).
    scale: multiplies Q K^T.  causal: keep key j <= query i.  seq_lens: None or B lengths
    (padding mask).  rows: None for every query row, or a 1-D list of row indices to
    compute (the definition is row-wise, so a subset is exact for those rows).

    Returns (O [B, H, n_rows, d] float64, LSE [B, H, n_rows] float64).
    """
    o, lse, _ = _attention(q, k, v, scale, causal, seq_lens, rows, want_probs=False)
    return o, lse


def attention_probs_ref(q, k, v, scale, causal=False, seq_lens=None, rows=None):
    """Same as attention_ref but also returns P [B, H, n_rows, N] (0 where invisible)."""
    return _attention(q, k, v, scale, causal, seq_lens, rows, want_probs=True)


def _attention(q, k, v, scale, causal, seq_lens, rows, want_probs):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Hkv, N, d = _check_shapes(q, k, v)
    group = H // Hkv
    lens = _lengths(seq_lens, B, N)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    if rows.size and (rows.min() < 0 or rows.max() >= N):
        raise ValueError("rows out of range")
    n = rows.size
    o = np.zeros((B, H, n, d))
    lse = np.full((B, H, n), -np.inf)
    probs = np.zeros((B, H, n, N)) if want_probs else None
    for b in range(B):
        L = lens[b]
        valid = rows < L                      # padded query rows keep O = 0, LSE = -inf
        if L == 0 or not valid.any():
            continue
        vr = rows[valid]
        counts = _visible_keys(vr, L, causal)
        for h in range(H):
            g = h // group
            ob, lb, pb = _three_pass(q[b, h, vr], k[b, g, :L], v[b, g, :L], float(scale), counts)
            o[b, h, valid] = ob
            lse[b, h, valid] = lb
            if want_probs:
                probs[b, h, np.flatnonzero(valid), :L] = pb
    return o, lse, probs
