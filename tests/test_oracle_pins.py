"""Pins for the fp64 oracle, each against something other than the oracle itself.

Closed forms (equal scores, scale 0, causal row 0, two keys, one-hot values), invariances
(joint key/value permutation, a shift of every key by one vector, GQA versus repeated-KV
multi-head, paged versus contiguous, block relabelling), a pure-Python brute force on tiny
inputs, an independent blockwise online-softmax recurrence, and two library routines
(torch's float64 scaled_dot_product_attention / logsumexp and scipy's softmax).
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import expit, logsumexp, softmax

from oracle import attention_probs_ref, attention_ref, gather_paged_kv, paged_decode_ref


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_equal_scores_give_mean_of_values(causal):
    rng = np.random.default_rng(11)
    B, H, N, d = 2, 3, 13, 8
    q = _rand(rng, B, H, N, d)
    k = np.broadcast_to(_rand(rng, B, H, 1, d), (B, H, N, d)).copy()   # every key row equal
    v = _rand(rng, B, H, N, d)
    scale = 0.37
    o, lse = attention_ref(q, k, v, scale, causal=causal)
    s = scale * np.einsum("bhnd,bhd->bhn", q, k[:, :, 0])                 # the one score per row
    if causal:
        counts = np.arange(1, N + 1)
        mean = np.cumsum(v, axis=2) / counts[None, None, :, None]
    else:
        counts = np.full(N, N)
        mean = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    np.testing.assert_allclose(o, mean, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, s + np.log(counts)[None, None, :], rtol=0, atol=1e-12)


def test_zero_query_and_zero_scale_give_log_n():
    rng = np.random.default_rng(12)
    B, H, N, d = 1, 2, 17, 4
    k = _rand(rng, B, H, N, d)
    v = _rand(rng, B, H, N, d)
    for q, scale in ((np.zeros((B, H, N, d)), 0.5), (_rand(rng, B, H, N, d), 0.0)):
        o, lse = attention_ref(q, k, v, scale)
        np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape),
                                   atol=1e-12)
        np.testing.assert_allclose(lse, np.full((B, H, N), math.log(N)), atol=1e-12)


def test_rows_of_p_sum_to_one_and_masked_entries_are_zero():
    rng = np.random.default_rng(13)
    B, H, N, d = 2, 2, 19, 8
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    lens = [19, 7]
    _, _, p = attention_probs_ref(q, k, v, 0.3, causal=True, seq_lens=lens)
    for b, L in enumerate(lens):
        np.testing.assert_allclose(p[b, :, :L].sum(axis=-1), 1.0, atol=1e-12)
        assert (p[b] >= 0).all()
        i, j = np.meshgrid(np.arange(N), np.arange(N), indexing="ij")
        assert (p[b][:, (j > i) | (j >= L)] == 0).all()
        assert (p[b, :, L:] == 0).all()


def test_one_hot_values_select_columns_of_p():
    rng = np.random.default_rng(14)
    N = d = 8
    q, k = _rand(rng, 1, 1, N, d), _rand(rng, 1, 1, N, d)
    v = np.eye(N)[None, None]                                   # value row j is e_j
    scale = 0.9
    o, _ = attention_ref(q, k, v, scale)
    # library softmax of the scores, independent of the oracle
    p = softmax(scale * q[0, 0] @ k[0, 0].T, axis=1)
    np.testing.assert_allclose(o[0, 0], p, atol=1e-13)
    # a single one-hot column picks one column of P
    for j in (0, 5):
        vj = np.zeros((1, 1, N, d))
        vj[0, 0, j, 3] = 1.0
        oj, _ = attention_ref(q, k, vj, scale)
        np.testing.assert_allclose(oj[0, 0, :, 3], p[:, j], atol=1e-13)
        np.testing.assert_allclose(np.delete(oj[0, 0], 3, axis=1), 0.0, atol=0)


def test_causal_row_zero_returns_first_value():
    rng = np.random.default_rng(15)
    q, k, v = (_rand(rng, 2, 2, 9, 16) for _ in range(3))
    o, lse = attention_ref(q, k, v, 0.25, causal=True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.25 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               atol=1e-13)


def test_two_keys_give_a_sigmoid():
    rng = np.random.default_rng(16)
    q, k, v = (_rand(rng, 1, 1, 2, 4) for _ in range(3))
    scale = 0.7
    o, lse = attention_ref(q, k, v, scale)
    s = scale * q[0, 0] @ k[0, 0].T                            # [2 queries, 2 keys]
    w0 = expit(s[:, 0] - s[:, 1])
    expect = w0[:, None] * v[0, 0, 0] + (1 - w0)[:, None] * v[0, 0, 1]
    np.testing.assert_allclose(o[0, 0], expect, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.logaddexp(s[:, 0], s[:, 1]), atol=1e-13)


# ---------------------------------------------------------------------------------------------
# invariances
# ---------------------------------------------------------------------------------------------

def test_joint_key_value_permutation_is_invisible():
    rng = np.random.default_rng(21)
    q, k, v = (_rand(rng, 1, 2, 23, 8) for _ in range(3))
    perm = rng.permutation(23)
    o1, l1 = attention_ref(q, k, v, 0.4)
    o2, l2 = attention_ref(q, k[:, :, perm], v[:, :, perm], 0.4)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_shifting_every_key_shifts_lse_only(causal):
    rng = np.random.default_rng(22)
    q, k, v = (_rand(rng, 1, 2, 15, 8) for _ in range(3))
    u = _rand(rng, 8)
    scale = 0.6
    o1, l1 = attention_ref(q, k, v, scale, causal=causal)
    o2, l2 = attention_ref(q, k + u, v, scale, causal=causal)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + scale * (q @ u), atol=1e-12)


def test_gqa_equals_multi_head_with_repeated_kv():
    rng = np.random.default_rng(23)
    B, H, Hkv, N, d = 2, 8, 2, 11, 8
    q = _rand(rng, B, H, N, d)
    k, v = _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    o1, l1 = attention_ref(q, k, v, 0.3, causal=True, seq_lens=[11, 6])
    rep = H // Hkv
    o2, l2 = attention_ref(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), 0.3,
                           causal=True, seq_lens=[11, 6])
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_padding_rows_and_truncation():
    rng = np.random.default_rng(24)
    q, k, v = (_rand(rng, 2, 2, 20, 8) for _ in range(3))
    lens = [20, 9]
    for causal in (False, True):
        o, l = attention_ref(q, k, v, 0.35, causal=causal, seq_lens=lens)
        assert (o[1, :, 9:] == 0).all() and np.isneginf(l[1, :, 9:]).all()
        ot, lt = attention_ref(q[1:, :, :9], k[1:, :, :9], v[1:, :, :9], 0.35, causal=causal)
        np.testing.assert_allclose(o[1, :, :9], ot[0], atol=1e-12)
        np.testing.assert_allclose(l[1, :, :9], lt[0], atol=1e-12)


def test_row_subset_matches_full_rows():
    rng = np.random.default_rng(25)
    q, k, v = (_rand(rng, 1, 2, 33, 8) for _ in range(3))
    rows = [0, 5, 31, 32]
    o, l = attention_ref(q, k, v, 0.2, causal=True, seq_lens=[30])
    os_, ls_ = attention_ref(q, k, v, 0.2, causal=True, seq_lens=[30], rows=rows)
    np.testing.assert_array_equal(o[:, :, rows], os_)
    np.testing.assert_array_equal(l[:, :, rows], ls_)


# ---------------------------------------------------------------------------------------------
# brute force in pure Python (no numpy arithmetic)
# ---------------------------------------------------------------------------------------------

def _brute(q, k, v, scale, causal, lens, group):
    B, H, N, d = q.shape
    o = [[[[0.0] * d for _ in range(N)] for _ in range(H)] for _ in range(B)]
    lse = [[[-math.inf] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        L = lens[b]
        for h in range(H):
            g = h // group
            for i in range(min(L, N)):
                keys = [j for j in range(L) if (not causal or j <= i)]
                s = [scale * math.fsum(float(q[b, h, i, t]) * float(k[b, g, j, t]) for t in range(d))
                     for j in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                for t in range(d):
                    o[b][h][i][t] = math.fsum(wj * float(v[b, g, j, t]) for wj, j in zip(w, keys)) / tot
                lse[b][h][i] = mx + math.log(tot)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1), (1, 2, 2, 7, 4), (2, 4, 2, 16, 8)])
def test_brute_force_tiny(causal, shape):
    B, H, Hkv, N, d = shape
    rng = np.random.default_rng(31 + N)
    q = _rand(rng, B, H, N, d)
    k, v = _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    lens = [N] * B if B == 1 else [N, max(1, N // 3)]
    o, l = attention_ref(q, k, v, 0.45, causal=causal, seq_lens=lens)
    ob, lb = _brute(q, k, v, 0.45, causal, lens, H // Hkv)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(l, lb, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# library routines
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    rng = np.random.default_rng(41)
    B, H, Hkv, N, d = 2, 8, 2, 40, 16
    q = _rand(rng, B, H, N, d)
    k, v = _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    lens = [40, 23]
    scale = 1 / math.sqrt(d)
    o, l = attention_ref(q, k, v, scale, causal=causal, seq_lens=lens)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    for b, L in enumerate(lens):
        allowed = (j < L) & ((j <= i) if causal else torch.ones_like(j <= i))
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq[b:b + 1], tk[b:b + 1], tv[b:b + 1], attn_mask=allowed, scale=scale, enable_gqa=True)
        np.testing.assert_allclose(o[b, :, :L], ref[0, :, :L].numpy(), atol=1e-12)
        kk = torch.repeat_interleave(tk[b], H // Hkv, dim=0)
        s = scale * tq[b] @ kk.transpose(-1, -2)
        s = s.masked_fill(~allowed, float("-inf"))
        np.testing.assert_allclose(l[b, :, :L], torch.logsumexp(s, dim=-1)[:, :L].numpy(), atol=1e-12)


def test_online_blockwise_recurrence_any_order():
    """The running max / running sum recurrence ("FlashAttention优化" §3.2.1), done blockwise in
    a shuffled block order, reaches the oracle's result (the §3.2.2 exactness claim)."""
    rng = np.random.default_rng(42)
    N, d, bs = 64, 8, 8
    q, k, v = (_rand(rng, 1, 1, N, d) for _ in range(3))
    scale = 0.5
    o_ref, l_ref = attention_ref(q, k, v, scale)
    order = rng.permutation(N // bs)
    for i in range(N):
        m, ell, acc = -math.inf, 0.0, np.zeros(d)
        for blk in order:
            js = range(blk * bs, (blk + 1) * bs)
            x = [scale * float(q[0, 0, i] @ k[0, 0, j]) for j in js]
            m_new = max(m, max(x))
            alpha = math.exp(m - m_new) if m > -math.inf else 0.0
            w = [math.exp(t - m_new) for t in x]
            ell = alpha * ell + math.fsum(w)
            acc = alpha * acc + sum(wj * v[0, 0, j] for wj, j in zip(w, js))
            m = m_new
        np.testing.assert_allclose(acc / ell, o_ref[0, 0, i], atol=1e-12)
        assert abs(m + math.log(ell) - l_ref[0, 0, i]) < 1e-12


# ---------------------------------------------------------------------------------------------
# paged decode
# ---------------------------------------------------------------------------------------------

def _paged_case(rng, S, Hq, Hkv, d, bs, lens, spare=3):
    nb = [-(-L // bs) for L in lens]
    P = sum(nb) + spare
    perm = rng.permutation(P)
    table = np.full((S, max(1, max(nb))), -1, dtype=np.int64)
    pos = 0
    for b, n in enumerate(nb):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    q = _rand(rng, S, Hq, d)
    kc, vc = _rand(rng, P, bs, Hkv, d), _rand(rng, P, bs, Hkv, d)
    return q, kc, vc, table


def test_gather_follows_the_block_table():
    rng = np.random.default_rng(51)
    q, kc, vc, table = _paged_case(rng, 2, 4, 2, 8, 4, [9, 4])
    g = gather_paged_kv(kc, table[0], 9)
    for t in range(9):
        np.testing.assert_array_equal(g[t], kc[table[0, t // 4], t % 4])


def test_paged_decode_equals_last_row_of_causal_attention():
    rng = np.random.default_rng(52)
    S, Hq, Hkv, d, bs = 3, 8, 2, 16, 4
    lens = [1, 13, 16]
    q, kc, vc, table = _paged_case(rng, S, Hq, Hkv, d, bs, lens)
    o, l = paged_decode_ref(q, kc, vc, table, lens, 0.25)
    for b, L in enumerate(lens):
        kb = gather_paged_kv(kc, table[b], L).transpose(1, 0, 2)[None]   # [1, Hkv, L, d]
        vb = gather_paged_kv(vc, table[b], L).transpose(1, 0, 2)[None]
        qq = _rand(rng, 1, Hq, L, d)
        qq[0, :, L - 1] = q[b]
        oc, lc = attention_ref(qq, kb, vb, 0.25, causal=True, rows=[L - 1])
        np.testing.assert_allclose(o[b], oc[0, :, 0], atol=1e-12)
        np.testing.assert_allclose(l[b], lc[0, :, 0], atol=1e-12)


def test_paged_decode_block_relabelling_is_bitwise_invisible():
    rng = np.random.default_rng(53)
    S, Hq, Hkv, d, bs = 2, 4, 1, 8, 4
    lens = [11, 6]
    q, kc, vc, table = _paged_case(rng, S, Hq, Hkv, d, bs, lens, spare=0)
    relabel = rng.permutation(kc.shape[0])
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[relabel] = kc
    vc2[relabel] = vc
    table2 = np.where(table >= 0, relabel[np.maximum(table, 0)], -1)
    o1, l1 = paged_decode_ref(q, kc, vc, table, lens, 0.3)
    o2, l2 = paged_decode_ref(q, kc2, vc2, table2, lens, 0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_paged_decode_brute_force_and_empty_sequence():
    rng = np.random.default_rng(54)
    S, Hq, Hkv, d, bs = 3, 4, 2, 4, 4
    lens = [5, 0, 3]
    q, kc, vc, table = _paged_case(rng, S, Hq, Hkv, d, bs, lens)
    o, l = paged_decode_ref(q, kc, vc, table, lens, 0.8)
    assert (o[1] == 0).all() and np.isneginf(l[1]).all()
    for b, L in enumerate(lens):
        for h in range(Hq):
            if L == 0:
                continue
            g = h // (Hq // Hkv)
            rowsk = [kc[table[b, t // bs], t % bs, g] for t in range(L)]
            rowsv = [vc[table[b, t // bs], t % bs, g] for t in range(L)]
            s = [0.8 * math.fsum(float(a) * float(c) for a, c in zip(q[b, h], r)) for r in rowsk]
            lse = float(logsumexp(s))
            w = [math.exp(x - lse) for x in s]
            for t in range(d):
                assert abs(o[b, h, t] - math.fsum(wj * float(r[t]) for wj, r in zip(w, rowsv))) < 1e-12
            assert abs(l[b, h] - lse) < 1e-12


# ---------------------------------------------------------------------------------------------
# chunked prefill against the paged cache
# ---------------------------------------------------------------------------------------------

def test_paged_prefill_equals_the_last_rows_of_causal_attention():
    # The chunk's rows are the last Q rows of causal attention over the whole gathered sequence.
    from oracle import paged_prefill_ref
    rng = np.random.default_rng(55)
    S, Hq, Hkv, d, bs = 3, 4, 2, 8, 4
    lens, qls, Qmax = [13, 7, 16], [5, 6, 1], 6
    _, kc, vc, table = _paged_case(rng, S, Hq, Hkv, d, bs, lens)
    q = _rand(rng, S, Hq, Qmax, d)
    o, l = paged_prefill_ref(q, kc, vc, table, lens, qls, 0.3)
    for b, (L, Q) in enumerate(zip(lens, qls)):
        kb = gather_paged_kv(kc, table[b], L).transpose(1, 0, 2)[None]   # [1, Hkv, L, d]
        vb = gather_paged_kv(vc, table[b], L).transpose(1, 0, 2)[None]
        qq = _rand(rng, 1, Hq, L, d)
        qq[0, :, L - Q:] = q[b, :, :Q]
        oc, lc = attention_ref(qq, kb, vb, 0.3, causal=True, rows=list(range(L - Q, L)))
        np.testing.assert_allclose(o[b, :, :Q], oc[0], atol=1e-12)
        np.testing.assert_allclose(l[b, :, :Q], lc[0], atol=1e-12)
        assert not o[b, :, Q:].any() and np.isneginf(l[b, :, Q:]).all()


def test_paged_prefill_of_one_token_is_a_decode_step():
    from oracle import paged_prefill_ref
    rng = np.random.default_rng(56)
    S, Hq, Hkv, d, bs = 3, 8, 2, 16, 4
    lens = [1, 13, 16]
    q, kc, vc, table = _paged_case(rng, S, Hq, Hkv, d, bs, lens)
    od, ld = paged_decode_ref(q, kc, vc, table, lens, 0.25)
    op, lp = paged_prefill_ref(q[:, :, None, :], kc, vc, table, lens, [1, 1, 1], 0.25)
    np.testing.assert_allclose(op[:, :, 0], od, atol=1e-12)
    np.testing.assert_allclose(lp[:, :, 0], ld, atol=1e-12)


@pytest.mark.parametrize("rows", [[0, 5, 1], [2, 3, 4, 5]])
def test_paged_prefill_row_subset_matches_full_rows(rows):
    # Rows of each sequence's chunk (and rows past a chunk, which are padding) equal the same rows
    # of the full computation.
    from oracle import paged_prefill_ref
    rng = np.random.default_rng(57)
    S, Hq, Hkv, d, bs = 4, 4, 2, 8, 4
    lens, qls, Qmax = [13, 7, 16, 0], [5, 6, 1, 0], 6
    _, kc, vc, table = _paged_case(rng, S, Hq, Hkv, d, bs, lens)
    q = _rand(rng, S, Hq, Qmax, d)
    o, l = paged_prefill_ref(q, kc, vc, table, lens, qls, 0.3)
    os_, ls_ = paged_prefill_ref(q, kc, vc, table, lens, qls, 0.3, rows=rows)
    np.testing.assert_array_equal(os_, o[:, :, rows])
    np.testing.assert_array_equal(ls_, l[:, :, rows])
