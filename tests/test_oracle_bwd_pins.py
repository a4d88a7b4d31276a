"""Pins for the fp64 backward oracle, each against something other than its own formulas.

* Central finite differences of the (separately pinned) forward oracle: the gradient of the
  scalar sum(O * dO) with respect to every element of Q, K and V.
* A library routine: torch's float64 autograd through scaled_dot_product_attention (CPU).
* Closed forms: dO = 0; scale 0 (uniform probabilities); causal row 0 (one visible key).
* Invariances: dQ unchanged when every key is shifted by one vector (each row of dS sums to
  zero); grouped-query heads equal multi-head attention on repeated K/V with the repeated
  heads' dK, dV summed; padding rows and keys get zero gradients and do not affect the rest.
"""

import numpy as np
import pytest
import torch

from oracle import attention_bwd_ref, attention_ref


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _loss(q, k, v, do, scale, causal, seq_lens):
    o, _ = attention_ref(q, k, v, scale, causal=causal, seq_lens=seq_lens)
    return float((o * do[:, :, : o.shape[2]]).sum())


@pytest.mark.parametrize("causal,lens", [(False, None), (True, None), (True, [4, 5]),
                                         (False, [3, 5])])
def test_matches_central_finite_differences(causal, lens):
    rng = np.random.default_rng(21)
    B, H, Hkv, N, d = 2, 2, 1, 5, 3
    q, k, v = _rand(rng, B, H, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    do = _rand(rng, B, H, N, d)
    scale = 0.7
    dq, dk, dv = attention_bwd_ref(q, k, v, do, scale, causal=causal, seq_lens=lens)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            up = _loss(q, k, v, do, scale, causal, lens)
            x[idx] = keep - h
            dn = _loss(q, k, v, do, scale, causal, lens)
            x[idx] = keep
            num[idx] = (up - dn) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_float64(causal):
    rng = np.random.default_rng(22)
    B, H, N, d = 2, 3, 33, 16
    q, k, v, do = (_rand(rng, B, H, N, d) for _ in range(4))
    scale = 0.25
    dq, dk, dv = attention_bwd_ref(q, k, v, do, scale, causal=causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=0, atol=1e-11)


def test_zero_output_gradient_gives_zero():
    rng = np.random.default_rng(23)
    q, k, v = (_rand(rng, 1, 2, 9, 4) for _ in range(3))
    for g in attention_bwd_ref(q, k, v, np.zeros_like(q), 0.5, causal=True):
        assert not g.any()


def test_scale_zero_gives_uniform_weights():
    # S = 0: P = 1/N in every row, so dV_j = mean_i dO_i and dQ = dK = 0 (both carry the scale).
    rng = np.random.default_rng(24)
    B, H, N, d = 1, 2, 11, 5
    q, k, v, do = (_rand(rng, B, H, N, d) for _ in range(4))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, 0.0)
    assert not dq.any() and not dk.any()
    np.testing.assert_allclose(dv, np.broadcast_to(do.mean(axis=2, keepdims=True), dv.shape),
                               rtol=0, atol=1e-12)


def test_causal_row_zero_has_no_query_gradient():
    # Row 0 sees only key 0: its probability is 1 whatever q_0 or k_0 are, so dQ_0 = 0.  With an
    # output gradient on row 0 alone, dV_0 = dO_0 exactly and every other gradient is zero.
    rng = np.random.default_rng(25)
    N, d = 7, 4
    q, k, v, do = (_rand(rng, 1, 1, N, d) for _ in range(4))
    dq, _, _ = attention_bwd_ref(q, k, v, do, 0.6, causal=True)
    np.testing.assert_allclose(dq[0, 0, 0], 0.0, atol=1e-13)
    row0 = np.where(np.arange(N)[None, None, :, None] == 0, do, 0.0)
    dq, dk, dv = attention_bwd_ref(q, k, v, row0, 0.6, causal=True)
    np.testing.assert_allclose(dv[0, 0, 0], do[0, 0, 0], rtol=0, atol=1e-13)
    assert not dv[0, 0, 1:].any()
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, atol=1e-13)


def test_query_gradient_ignores_a_shift_of_every_key():
    rng = np.random.default_rng(26)
    B, H, N, d = 1, 2, 12, 6
    q, k, v, do = (_rand(rng, B, H, N, d) for _ in range(4))
    u = _rand(rng, 1, 1, 1, d)
    a = attention_bwd_ref(q, k, v, do, 0.4)
    b = attention_bwd_ref(q, k + u, v, do, 0.4)
    np.testing.assert_allclose(b[0], a[0], rtol=0, atol=1e-11)   # dQ
    np.testing.assert_allclose(b[2], a[2], rtol=0, atol=1e-11)   # dV (P unchanged)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_query_equals_repeated_kv(causal):
    rng = np.random.default_rng(27)
    B, H, Hkv, N, d = 2, 6, 2, 10, 4
    q, do = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d)
    k, v = _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, 0.5, causal=causal)
    rep = H // Hkv
    dq2, dk2, dv2 = attention_bwd_ref(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), do,
                                      0.5, causal=causal)
    np.testing.assert_allclose(dq, dq2, atol=1e-12)
    np.testing.assert_allclose(dk, dk2.reshape(B, Hkv, rep, N, d).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dv, dv2.reshape(B, Hkv, rep, N, d).sum(axis=2), atol=1e-12)


def test_padding_is_inert():
    # Rows and keys past the length get zero gradients, and the valid part equals the
    # unpadded problem of length L.
    rng = np.random.default_rng(28)
    B, H, N, d, L = 1, 2, 9, 4, 6
    q, k, v, do = (_rand(rng, B, H, N, d) for _ in range(4))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, 0.5, causal=True, seq_lens=[L])
    assert not dq[:, :, L:].any() and not dk[:, :, L:].any() and not dv[:, :, L:].any()
    ref = attention_bwd_ref(q[:, :, :L], k[:, :, :L], v[:, :, :L], do[:, :, :L], 0.5, causal=True)
    for got, want in zip((dq, dk, dv), ref):
        np.testing.assert_allclose(got[:, :, :L], want, atol=1e-13)


@pytest.mark.parametrize("causal,lens", [(False, None), (True, [7, 10])])
def test_row_subset_equals_full_query_gradient(causal, lens):
    rng = np.random.default_rng(29)
    B, H, Hkv, N, d = 2, 4, 2, 10, 5
    q, do = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d)
    k, v = _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    full, _, _ = attention_bwd_ref(q, k, v, do, 0.3, causal=causal, seq_lens=lens)
    rows = [9, 0, 4, 7]
    sub, dk, dv = attention_bwd_ref(q, k, v, do, 0.3, causal=causal, seq_lens=lens, rows=rows)
    assert dk is None and dv is None
    np.testing.assert_allclose(sub, full[:, :, rows], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,lens", [(False, None), (True, [7, 10]), (True, [0, 9])])
def test_key_subset_equals_full_key_gradients(causal, lens):
    # dK, dV of selected keys (grouped heads summed, keys past a length zero) equal the same
    # rows of the full computation, whichever way the query rows are blocked.
    from oracle.backward import _dkdv_keys
    rng = np.random.default_rng(30)
    B, H, Hkv, N, d = 2, 6, 2, 10, 5
    q, do = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d)
    k, v = _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    _, fk, fv = attention_bwd_ref(q, k, v, do, 0.3, causal=causal, seq_lens=lens)
    keys = [9, 0, 4, 7, 8]
    dq, dk, dv = attention_bwd_ref(q, k, v, do, 0.3, causal=causal, seq_lens=lens, keys=keys)
    assert dq is None
    np.testing.assert_allclose(dk, fk[:, :, keys], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, fv[:, :, keys], rtol=0, atol=1e-13)
    for blk in (1, 3, 4):
        bk, bv = _dkdv_keys(q, k, v, do, 0.3, causal, lens, keys, row_block=blk)
        np.testing.assert_allclose(bk, fk[:, :, keys], rtol=0, atol=1e-13)
        np.testing.assert_allclose(bv, fv[:, :, keys], rtol=0, atol=1e-13)
