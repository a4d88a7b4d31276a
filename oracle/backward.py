"""Attention backward in float64, materialised (oracle; test infrastructure).

What it computes: the gradients of the forward definition in ``oracle/attention.py`` --
O = P V with P the row softmax of S = scale * Q K^T (the "GPU优化" tag page, excerpt "Flash
Attention解决了什么问题？", 标准注意力计算) -- with respect to Q, K and V, for a given output
gradient dO.  They are the chain rule written out, with the full probability matrix in memory:

    dV = P^T dO                       (O is linear in V)
    dP = dO V^T                       (O is linear in P)
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)
                                      (the derivative of a row softmax: for p = softmax(s),
                                       dL/ds = p o (dL/dp - <p, dL/dp>))
    dQ = scale * dS K,   dK = scale * dS^T Q
                                      (S = scale * Q K^T is bilinear in Q and K)

The fused kernel never stores P: it rebuilds it from the per-row log-sum-exp the forward
wrote ("Gemini 3 Flash的注意力内核重写" §4 on recomputation).  This oracle materialises P with
the forward oracle's three passes instead, so it shares nothing with that recomputation.

Grouped-query heads: kv head g receives the sum of the gradients of the query heads that read
it.  Padding (per-sequence length L_b): query rows i >= L_b get dQ = 0, keys j >= L_b get
dK = dV = 0 (they take no part in any visible score).
"""

import numpy as np

from .attention import _check_shapes, _lengths, _three_pass, _visible_keys

__all__ = ["attention_bwd_ref"]


def attention_bwd_ref(q, k, v, dout, scale, causal=False, seq_lens=None, rows=None, keys=None):
    """Gradients (dQ [B,H,N,d], dK [B,Hkv,N,d], dV [B,Hkv,N,d]) in float64.

    q, dout [B, H, N, d]; k, v [B, Hkv, N, d] (any real dtype; upcast exactly to float64).
    scale, causal and seq_lens as for ``attention_ref``.  With ``rows`` (a 1-D list of query
    rows) only dQ of those rows is computed -- dQ_i needs row i of P alone -- and the result is
    (dQ [B, H, n_rows, d], None, None).  With ``keys`` (a 1-D list of key rows) only dK and dV
    of those keys are computed and the result is (None, dK [B, Hkv, n_keys, d],
    dV [B, Hkv, n_keys, d]); column j of P still needs every row's normaliser, so every query
    row of the sequence takes part.
    """
    if rows is not None and keys is not None:
        raise ValueError("give rows or keys, not both")
    if rows is not None:
        return _dq_rows(q, k, v, dout, scale, causal, seq_lens, rows), None, None
    if keys is not None:
        dk, dv = _dkdv_keys(q, k, v, dout, scale, causal, seq_lens, keys)
        return None, dk, dv
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    B, H, Hkv, N, d = _check_shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    group = H // Hkv
    lens = _lengths(seq_lens, B, N)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    scale = float(scale)
    for b in range(B):
        L = lens[b]
        if L == 0:
            continue
        rows = np.arange(L)
        counts = _visible_keys(rows, L, causal)
        for h in range(H):
            g = h // group
            qb, kb, vb, dob = q[b, h, :L], k[b, g, :L], v[b, g, :L], do[b, h, :L]
            _, _, p = _three_pass(qb, kb, vb, scale, counts)    # P [L, L], 0 where invisible
            dv[b, g, :L] += p.T @ dob
            dp = dob @ vb.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, h, :L] = scale * (ds @ kb)
            dk[b, g, :L] += scale * (ds.T @ qb)
    return dq, dk, dv


def _dq_rows(q, k, v, dout, scale, causal, seq_lens, rows):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    B, H, Hkv, N, d = _check_shapes(q, k, v)
    group = H // Hkv
    lens = _lengths(seq_lens, B, N)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    dq = np.zeros((B, H, rows.size, d))
    scale = float(scale)
    for b in range(B):
        L = lens[b]
        valid = rows < L
        if L == 0 or not valid.any():
            continue
        vr = rows[valid]
        counts = _visible_keys(vr, L, causal)
        for h in range(H):
            g = h // group
            _, _, p = _three_pass(q[b, h, vr], k[b, g, :L], v[b, g, :L], scale, counts)
            dp = do[b, h, vr] @ v[b, g, :L].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, h, valid] = scale * (ds @ k[b, g, :L])
    return dq


def _dkdv_keys(q, k, v, dout, scale, causal, seq_lens, keys, row_block=2048):
    """dK and dV of the key rows ``keys`` only.

    Column j of P is exp(S_:j - LSE), so every query row's log-sum-exp is needed: each row's
    softmax is formed with the three passes of the forward oracle (in blocks of query rows, to
    bound memory; the rows are independent).  The row term of the softmax derivative is
    sum_k P_ik dP_ik = dO_i . O_i, where O_i = sum_k P_ik V_k is the same three-pass output,
    so the full dP matrix is not needed.  Then for the selected columns J:
        dP_:J = dO V_J^T,  dS_:J = P_:J o (dP_:J - D),  dV_J = P_:J^T dO,  dK_J = scale dS_:J^T Q
    summed over the query heads of each kv head and over the query rows.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    B, H, Hkv, N, d = _check_shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    group = H // Hkv
    lens = _lengths(seq_lens, B, N)
    keys = np.asarray(keys, dtype=np.int64).reshape(-1)
    if keys.size and (keys.min() < 0 or keys.max() >= N):
        raise ValueError("keys out of range")
    dk = np.zeros((B, Hkv, keys.size, d))
    dv = np.zeros((B, Hkv, keys.size, d))
    scale = float(scale)
    for b in range(B):
        L = lens[b]
        valid = keys < L                   # keys past the length keep dK = dV = 0
        if L == 0 or not valid.any():
            continue
        kj = keys[valid]
        for h in range(H):
            g = h // group
            kb, vb = k[b, g, :L], v[b, g, :L]
            for r0 in range(0, L, row_block):
                rows = np.arange(r0, min(L, r0 + row_block))
                counts = _visible_keys(rows, L, causal)
                o, _, p = _three_pass(q[b, h, rows], kb, vb, scale, counts)   # P [n, L]
                dob = do[b, h, rows]
                drow = (dob * o).sum(axis=1)                                   # D_i = dO_i . O_i
                pj = p[:, kj]                                                  # P_:J
                dpj = dob @ vb[kj].T                                           # dP_:J
                dsj = pj * (dpj - drow[:, None])
                dv[b, g, valid] += pj.T @ dob
                dk[b, g, valid] += scale * (dsj.T @ q[b, h, rows])
    return dk, dv
