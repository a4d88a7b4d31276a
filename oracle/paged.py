"""Paged decode attention in float64 (oracle; test infrastructure).

Page "非连续块Gather" (ocdem.com, vLLM PagedAttention kernel rework) §二.1 and §二.3: the keys
and values of one sequence live in physical blocks scattered through a pool, found through an
index array.  This oracle gathers them back into a contiguous sequence, token by token, and
then applies the same three-pass softmax attention as ``attention.py`` with a single query row
that sees every cached token (the query is the newest token; "FlashAttention优化" §4.2.2
describes decode as one token against the O(N d) cache).

Layouts (readings of points the pages leave open):
* q        [S, Hq, d]
* k_cache  [num_blocks, block_size, Hkv, d]   (token-major inside a block)
* v_cache  same as k_cache
* block_table [S, max_blocks] integer physical block ids; entry t // block_size holds token t
* seq_lens [S]; a sequence of length 0 yields O = 0, LSE = -inf.
Query head h reads kv head h // (Hq // Hkv).

Chunked prefill against the cache (``paged_prefill_ref``): the query chunk of sequence b is its
newest Q_b tokens, positions L_b - Q_b .. L_b - 1, whose keys and values are already in the
cache; query i sees the cached tokens 0 .. L_b - Q_b + i (causal with that offset).  This is
the chunked prefill of "LLM inference optimisation" §3.2 (a long prompt processed in pieces
against the cache built so far); with Q_b = 1 it is one decode step.  Layout (head-major, as
the prefill forward): q [S, Hq, Qmax, d]; rows i >= Q_b are padding and get O = 0, LSE = -inf.
"""

import numpy as np

from .attention import _three_pass

__all__ = ["gather_paged_kv", "paged_decode_ref", "paged_prefill_ref"]


def gather_paged_kv(cache, block_table_row, length):
    """Contiguous [length, Hkv, d] float64 view of one sequence's tokens from a paged pool.

    Token t lives in physical block block_table_row[t // block_size] at slot t % block_size.
    """
    cache = np.asarray(cache)
    bs = cache.shape[1]
    t = np.arange(length)
    blocks = np.asarray(block_table_row, dtype=np.int64)[t // bs]
    if length and (blocks.min() < 0 or blocks.max() >= cache.shape[0]):
        raise ValueError("block id out of range")
    return cache[blocks, t % bs].astype(np.float64)


def paged_decode_ref(q, k_cache, v_cache, block_table, seq_lens, scale):
    """One decode step: O [S, Hq, d] and LSE [S, Hq] in float64."""
    q = np.asarray(q, dtype=np.float64)
    S, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    if k_cache.shape != v_cache.shape or k_cache.shape[3] != d or Hq % Hkv != 0:
        raise ValueError("inconsistent shapes")
    group = Hq // Hkv
    lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    o = np.zeros((S, Hq, d))
    lse = np.full((S, Hq), -np.inf)
    for b in range(S):
        L = lens[b]
        if L == 0:
            continue
        kb = gather_paged_kv(k_cache, block_table[b], L)    # [L, Hkv, d]
        vb = gather_paged_kv(v_cache, block_table[b], L)
        for h in range(Hq):
            g = h // group
            # pass 1: scores of the single query row and their maximum
            s = float(scale) * (kb[:, g, :] @ q[b, h])
            m = s.max()
            # pass 2: exponentials and their sum
            e = np.exp(s - m)
            l = e.sum()
            # pass 3: normalise and weight the values
            o[b, h] = (e / l) @ vb[:, g, :]
            lse[b, h] = m + np.log(l)
    return o, lse


def paged_prefill_ref(q, k_cache, v_cache, block_table, seq_lens, q_lens, scale, rows=None):
    """Chunked prefill: O [S, Hq, Qmax, d] and LSE [S, Hq, Qmax] in float64.

    rows: None for every query row, or a 1-D list of query-row indices (into Qmax) to compute;
    then the results are [S, Hq, n_rows, d] and [S, Hq, n_rows] (each row's softmax involves
    that row alone, so a subset is exact for those rows).  Rows at or past a sequence's chunk
    length are padding: O = 0, LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    S, Hq, Qmax, d = q.shape
    Hkv = k_cache.shape[2]
    if k_cache.shape != v_cache.shape or k_cache.shape[3] != d or Hq % Hkv != 0:
        raise ValueError("inconsistent shapes")
    group = Hq // Hkv
    lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    qls = [int(x) for x in np.asarray(q_lens).reshape(-1)]
    sel = np.arange(Qmax) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    if sel.size and (sel.min() < 0 or sel.max() >= Qmax):
        raise ValueError("rows out of range")
    o = np.zeros((S, Hq, sel.size, d))
    lse = np.full((S, Hq, sel.size), -np.inf)
    for b in range(S):
        L, Q = lens[b], qls[b]
        if Q > L or Q > Qmax:
            raise ValueError("q_lens must not exceed seq_lens or the query rows")
        valid = sel < Q
        if Q == 0 or not valid.any():
            continue
        kb = gather_paged_kv(k_cache, block_table[b], L)    # [L, Hkv, d]
        vb = gather_paged_kv(v_cache, block_table[b], L)
        counts = (L - Q) + sel[valid] + 1                    # keys visible to each query row
        for h in range(Hq):
            g = h // group
            ob, lb, _ = _three_pass(q[b, h, sel[valid]], kb[:, g, :], vb[:, g, :], float(scale),
                                    counts)
            o[b, h, valid] = ob
            lse[b, h, valid] = lb
    return o, lse
