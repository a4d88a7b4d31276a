"""Tolerance of the FP8 forward against the exact attention of its dequantised inputs.

The parity oracle for fa_fwd_fp8 is the plain definition: O = softmax(scale * Q K^T) V of the
tensors the e4m3 codes stand for (``oracle.attention_probs_ref`` on the decoded values).  The
pages fix no FP8 arithmetic (the "GPU优化" tag page, excerpt "注意力计算的性能瓶颈", FlashAttention
V3 part, names FP8 matrix cores only), so the kernel's deviation from that definition is bounded
from the e4m3 format and the way the probabilities enter the P V product:

* Rounding one probability.  The P V operand is e4m3(64 p) / 64 with p = exp(s - m) and m the
  row's reference.  The kernel's first pass fixes m at the maximum of the row's first 128 keys
  plus 2^4 and keeps only rows with 64 p <= 464 (a larger value has no e4m3 code and sends the
  workgroup to the second pass); its second pass keeps m at most the row maximum and at least
  2^-2 below the running one, so p <= 4.  Either way p <= 7.25 and max p >= 2^-4, and 64 p
  never saturates beyond rounding 448 < x <= 464 down to 448 (largest e4m3 value).  With 3
  mantissa bits, |e4m3(x) - x| <= 2^-4 * 2^floor(log2 x) <= 2^-4 x for x >= 2^-6 (normal
  numbers; also for 448 < x <= 464) and <= 2^-10 below (subnormal spacing 2^-9).  In units of
  the normalised probability P_j = p_j / l that is  delta_j = 2^-4 * max(P_j, 2^-8 * P_max),
  since 64 p_j >= 2^-6 iff p_j >= 2^-12 and 1 / l <= 2^4 P_max (because max p >= 2^-4).
* The rounding errors of different keys are bounded, zero-mean and independent -- the model of
  probabilistic rounding-error analysis (N. J. Higham and T. Mary, "A new approach to
  probabilistic rounding error analysis", SIAM J. Sci. Comput. 41(5), 2019).  Hoeffding's
  inequality bounds their weighted sum over keys: P(|sum_j e_j V_jc| > t) <=
  2 exp(-t^2 / (2 sum_j (delta_j V_jc)^2)); t = 8 * sqrt(sum_j (delta_j V_jc)^2) leaves
  2.5e-14 per output element.
* Scores.  Each score is a sum of exact products of e4m3 values; the tolerance allows it an
  error of E = 2^-7 in natural-log units (the LSE check, 1e-3, holds the average far tighter).
  A score error e_j changes O by sum_j P_j (e^{e_j} - 1)(V_j - O); its terms, bounded by
  (e^E - 1) P_j |V_j - O|, join the same Hoeffding sum.
* Accumulation of P V on the matrix cores: an allowance of 2^-10 * sum_j P_j |V_j| (the format
  does not fix the internal accumulation precision of the FP8 matrix cores).
* Output rounding to bf16: at most 2^-8 |O| (8 significand bits).

Two checks follow.  Element by element, |O - O_exact| must stay under the sum of these terms.
In aggregate, the mean of the squared errors over a tensor must stay under the mean of their
variance bound: a uniform rounding error within +-delta has variance delta^2 / 3, so the
bound is sum_j (delta_j V_jc)^2 / 3 + score terms / 3 + (accumulation allowance)^2 +
(2^-8 |O|)^2 / 3.  A localised mistake (a key block dropped, a value row misplaced) can hide
inside the elementwise bound at large N, where each element sums thousands of keys, but it
raises the mean squared error well above its bound.

This module holds no attention arithmetic of its own beyond these bounds; P, V and O come from
the oracle.
"""

import numpy as np

SCORE_ALLOW = 2.0 ** -7     # allowed error of one score, natural-log units
SUBNORMAL_FLOOR = 2.0 ** -8  # 2^-12 (64 p subnormal) times 2^4 (max p >= 2^-4), relative to P_max
HOEFFDING_T = 8.0           # t / sigma of the elementwise bound
ACC_ALLOW = 2.0 ** -10      # P V accumulation allowance, relative to sum_j P_j |V_j|
BF16_HALF_ULP = 2.0 ** -8   # output rounding, relative


def fp8_bounds(p, v, o):
    """Per-element bound and variance bound of |O_kernel - O_exact| for one (batch, head).

    p [n, L]: exact probabilities of n query rows (0 where invisible); v [L, d]: the dequantised
    values; o [n, d]: exact output.  Returns (bound [n, d], variance [n, d]).
    """
    p = np.asarray(p, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    pmax = p.max(axis=1, keepdims=True)
    delta = 2.0 ** -4 * np.where(p > 0, np.maximum(p, SUBNORMAL_FLOOR * pmax), 0.0)
    v2 = v * v
    rnd = (delta * delta) @ v2                                  # sum_j (delta_j V_jc)^2
    p2 = p * p
    spread = (p2 @ v2) - 2.0 * o * (p2 @ v) + o * o * p2.sum(axis=1, keepdims=True)
    scr = np.maximum(spread, 0.0) * np.expm1(SCORE_ALLOW) ** 2  # sum_j ((e^E-1) P_j |V_j-O|)^2
    acc = ACC_ALLOW * (p @ np.abs(v))
    rest = HOEFFDING_T * np.sqrt(rnd + scr) + acc
    bound = rest + BF16_HALF_ULP * (np.abs(o) + rest) + 1e-6
    var = (rnd + scr) / 3.0 + acc * acc + (BF16_HALF_ULP * np.abs(o)) ** 2 / 3.0
    return bound, var


def check_against_exact(go, ro, probs, v, group, lens=None, rows=None):
    """Compare kernel outputs with the exact attention of the dequantised inputs.

    go, ro [B, H, n, d] (kernel, exact), probs [B, H, n, N] (exact P of those rows), v
    [B, Hkv, N, d] dequantised values, ``group`` = H / Hkv.  ``rows`` are the query rows held in
    the n axis (None: all N); rows at or past a sequence's length are skipped here (their fill
    is checked by the caller).  Returns (worst elementwise error / bound, mean squared error /
    mean variance bound); raises AssertionError naming the first (batch, head) over the
    elementwise bound.
    """
    B, H, n, d = ro.shape
    N = v.shape[2]
    sel = np.arange(n) if rows is None else np.asarray(rows)
    worst, se, sv = 0.0, 0.0, 0.0
    for b in range(B):
        L = N if lens is None else int(lens[b])
        ok = sel < L
        if not ok.any():
            continue
        for h in range(H):
            bound, var = fp8_bounds(probs[b, h][ok][:, :L], v[b, h // group, :L], ro[b, h][ok])
            err = np.abs(go[b, h][ok] - ro[b, h][ok])
            assert np.isfinite(err).all(), f"({b},{h}): non-finite output"
            r = float(np.max(err / bound))
            assert r <= 1.0, f"({b},{h}): error {err.max():.3e} above the e4m3 bound (ratio {r:.2f})"
            worst = max(worst, r)
            se += float((err * err).sum())
            sv += float(var.sum())
    agg = se / sv if sv > 0 else 0.0
    return worst, agg
