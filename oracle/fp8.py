"""FP8 (e4m3) decoding, rounding, and a float64 model of rounded-probability attention
(oracle; test infrastructure).

The pages name FP8 as the main addition of FlashAttention V3 (the "GPU优化" tag page,
guijiagi.com, excerpt "注意力计算的性能瓶颈", part Flash Attention V3: FP8 tensor cores and an
asynchronous pipeline on the H100) without fixing the arithmetic.  What the FP8 path computes is
the exact attention of the dequantised tensors; its parity oracle is that definition (decode the
codes with ``e4m3_decode``, multiply by the descales, then the exact attention of
``attention.py``), and the tolerance against it is derived from the e4m3 format.  The function
``attention_fp8_ref`` below is NOT that oracle: it is a model of one way to round the
probabilities to e4m3 inside an online softmax, kept to check on the CPU that the derived
tolerance admits such rounding schemes (and rejects mistakes).  Its reading:

* Inputs are FP8 e4m3 codes (the OCP "fn" variant: 4 exponent bits with bias 7, 3 mantissa
  bits, no infinities, max 448) with one float descale factor per tensor: the real value of a
  code c of Q is ``q_scale * e4m3(c)`` (likewise K, V).
* The attention computed is the one of the dequantised tensors, O = softmax(scale * Q K^T) V,
  with the online softmax of "FlashAttention优化" (coreui.cn) §3.2.1: the keys are visited in
  blocks of ``block`` keys, a per-row reference m and sum l are kept, and the accumulated
  output and sum are rescaled by exp(m_old - m_new) whenever the reference moves.  The
  reference moves to a block's maximum only when that maximum exceeds it by more than
  ``lag`` (in log2 units, i.e. a factor 2^lag); lag = 0 is the plain running maximum.
* The probabilities of a block, p = exp(s - m) in (0, 2^lag], enter the P V product as FP8:
  ``e4m3_round(p_scale * p) / p_scale`` (p_scale = 64 with lag = 2 keeps 64 p <= 256 inside
  the e4m3 range and small probabilities out of the subnormals).  The row sum l uses the
  unrounded p, so the LSE is the exact log-sum-exp of the scaled scores.
* Optionally (``headroom``) the reference is fixed after the first ``first`` keys: the blocks
  among them use the lagging reference, then m becomes their maximum + headroom (log2 units),
  the output and sum are rescaled once, and later blocks keep it.  Every p then lies in
  (0, 2^headroom] below the row's largest one, which is at least 2^-headroom.  A row in which
  some ``p_scale * p`` would exceed 464 (no e4m3 code: the conversion gives NaN) is computed
  with the lagging reference throughout instead.

Because the rounding of p happens relative to the running maximum of each block, the result
depends on the block size and the lag; the model takes both as arguments, and any choice is one
admissible rounding scheme, not a specification of a kernel.  With ``p_scale=None`` nothing is
rounded and the function is the exact attention of the dequantised inputs (pinned against the
three-pass oracle).

e4m3 decoding and rounding are written out from the format's definition (no library cast).
"""

import numpy as np

from .attention import _check_shapes, _lengths, _visible_keys

__all__ = ["e4m3_decode", "e4m3_round", "attention_fp8_ref", "E4M3_MAX"]

E4M3_MAX = 448.0
_BIAS = 7
_MAN = 3


def e4m3_decode(codes):
    """Float64 values of e4m3fn byte codes (NaN for the two NaN codes 0x7f and 0xff)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> _MAN) & 0xF
    m = c & 0x7
    normal = sign * np.ldexp(1.0 + m / 8.0, e - _BIAS)
    sub = sign * np.ldexp(m / 8.0, 1 - _BIAS)          # exponent field 0: m/8 * 2^-6
    out = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_round(x):
    """Round float64 values to the nearest e4m3fn value, ties to the even mantissa.

    |x| must not exceed the largest finite value (448) by half a unit or more (no saturation
    is needed on the paths that use it: probabilities times 256 stay <= 256).
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    if np.any(ax >= E4M3_MAX + 16.0):  # 448 + half of the top spacing (32)
        raise ValueError("value outside the e4m3 range")
    # spacing of representable values around ax: 2^(e - 3) for normals (ax >= 2^-6), 2^-9 below
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, 1 - _BIAS)
    q = np.ldexp(1.0, (e - _MAN).astype(np.int64))
    n = ax / q
    r = np.floor(n)
    frac = n - r
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2) == 1))
    r = r + up
    return np.sign(x) * r * q


def attention_fp8_ref(q8, k8, v8, q_scale, k_scale, v_scale, scale, causal=False, seq_lens=None,
                      block=64, p_scale=64.0, lag=2.0, rows=None, headroom=None, first=128):
    """FP8 attention forward: (O [B, H, N, d], LSE [B, H, N]) in float64.

    q8 [B, H, N, d], k8 and v8 [B, Hkv, N, d]: e4m3 byte codes (uint8).  q_scale, k_scale,
    v_scale: per-tensor descale factors.  scale: the softmax scale of the scores.  causal,
    seq_lens, grouped-query heads and padding as for ``attention_ref``.  block: keys per block of
    the online softmax.  p_scale: the factor applied before rounding probabilities to e4m3, or
    None for no rounding.  lag: how far (log2 units) a block's maximum may exceed the row's
    reference before the reference moves.  headroom, first: None for the lagging reference on
    every block, else the reference is fixed after the first ``first`` keys (a multiple of
    ``block``) at their maximum + headroom (log2 units).  rows: None, or a 1-D list of query rows; then only those rows are
    computed (each row's recurrence involves that row alone) and the results are
    [B, H, n_rows, d] and [B, H, n_rows] (rows at or past a sequence's length: O = 0,
    LSE = -inf).
    """
    q = e4m3_decode(q8) * float(q_scale)
    k = e4m3_decode(k8) * float(k_scale)
    v = e4m3_decode(v8) * float(v_scale)
    B, H, Hkv, N, d = _check_shapes(q, k, v)
    group = H // Hkv
    lens = _lengths(seq_lens, B, N)
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    o = np.zeros((B, H, sel.size, d))
    lse = np.full((B, H, sel.size), -np.inf)
    for b in range(B):
        L = lens[b]
        valid = sel < L
        if L == 0 or not valid.any():
            continue
        counts = _visible_keys(sel[valid], L, causal)
        for h in range(H):
            g = h // group
            ob, lb = _online(q[b, h, sel[valid]], k[b, g, :L], v[b, g, :L], float(scale), counts,
                             block, p_scale, float(lag) * np.log(2.0), headroom, first)
            o[b, h, valid] = ob
            lse[b, h, valid] = lb
    return o, lse


def _online(qb, kb, vb, scale, counts, block, p_scale, lag, headroom=None, first=128):
    """Online softmax over key blocks for the rows of one sequence (every row sees >= 1 key).
    lag is in natural-log units here; headroom in log2 units (None: lagging reference only)."""
    n, L = qb.shape[0], kb.shape[0]
    s = scale * (qb @ kb.T)
    s = np.where(np.arange(L)[None, :] >= counts[:, None], -np.inf, s)
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, vb.shape[1]))
    fixed = None  # rows on the fixed reference: which rows, and the reference
    if headroom is not None:
        if first % block:
            raise ValueError("first must be a multiple of block")
        seen = s[:, :first].max(axis=1)
        ref = np.where(seen > -np.inf, seen, 0.0) + float(headroom) * np.log(2.0)
        # A row whose probabilities stay representable keeps the fixed reference.
        over = (p_scale is not None) & (s[:, first:].max(axis=1, initial=-np.inf) - ref
                                         >= np.log(464.0 / (p_scale or 1.0)))
        fixed = (~over, ref)
    for j0 in range(0, L, block):
        sj = s[:, j0:j0 + block]
        bm = sj.max(axis=1)
        if fixed is not None and j0 == first:
            keep, ref_f = fixed
            alpha_f = np.where(m > -np.inf, np.exp(np.where(m > -np.inf, m, 0.0) - ref_f), 0.0)
            acc = np.where(keep[:, None], alpha_f[:, None] * acc, acc)
            l = np.where(keep, alpha_f * l, l)
            m = np.where(keep, ref_f, m)
        lag_rows = np.ones(n, dtype=bool) if fixed is None or j0 < first else ~fixed[0]
        m_new = np.where(lag_rows & (bm > m + lag), bm, m)   # m = -inf: the first key sets it
        # rows with no visible key so far keep m = -inf and add nothing
        seen = m_new > -np.inf
        ref = np.where(seen, m_new, 0.0)
        alpha = np.where(seen, np.exp(np.where(seen, m - ref, 0.0)), 1.0)
        p = np.exp(sj - ref[:, None])                      # 0 where masked
        l = alpha * l + p.sum(axis=1)
        pq = p if p_scale is None else e4m3_round(p_scale * p) / p_scale
        acc = alpha[:, None] * acc + pq @ vb[j0:j0 + block]
        m = m_new
    return acc / l[:, None], m + np.log(l)
