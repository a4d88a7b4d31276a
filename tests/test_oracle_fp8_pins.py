"""Pins for the FP8 oracle, each against something other than its own formulas.

* A library routine: torch's float8_e4m3fn dtype for decoding all 256 codes and for rounding
  float32 values (including exact midpoints) to e4m3.
* Hand-derived e4m3 values (ties to even, subnormals, the largest finite value).
* The exact definition: with rounding switched off the online-softmax oracle equals the
  three-pass oracle (itself pinned against closed forms) for any block size, causal or not,
  with padding and grouped-query heads; the LSE never depends on the rounding.
* Closed forms: probabilities that are powers of two survive the rounding exactly; two keys
  with probabilities 1 and 0.3 give (V0 + 0.3125 V1) / 1.3 (64 * 0.3 = 19.2 rounds to 20);
  a reference that lags behind growing scores and then moves (hand-derived weights); equal
  scores give the mean of V; causal row 0 returns V[0].
* An error bound: the rounded result differs from the exact one by at most 2^-4 of the
  probability-weighted |V| per row (e4m3 keeps 3 mantissa bits).
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_fp8_ref, attention_ref, e4m3_decode, e4m3_round

F8 = torch.float8_e4m3fn


def _codes_of(values):
    """e4m3 codes of float32 values via torch (test-side helper for building inputs)."""
    return torch.tensor(np.asarray(values, dtype=np.float32)).to(F8).view(torch.uint8).numpy()


def test_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(F8).double().numpy()
    got = e4m3_decode(codes)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], want[~nan])


def test_round_matches_torch_cast():
    rng = np.random.default_rng(31)
    finite = np.unique(e4m3_decode(np.arange(256))[~np.isnan(e4m3_decode(np.arange(256)))])
    mids = (finite[1:] + finite[:-1]) / 2                        # exact ties
    rand = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(440.0), 4000)) * rng.choice([-1, 1], 4000)
    x = np.concatenate([finite, mids, rand]).astype(np.float32)  # all exact in float32
    x = x[np.abs(x) <= 448]
    want = torch.from_numpy(x).to(F8).double().numpy()
    np.testing.assert_array_equal(e4m3_round(x.astype(np.float64)), want)


@pytest.mark.parametrize("x,want", [(1.0625, 1.0), (1.1875, 1.25), (2.0 ** -10, 0.0),
                                    (3 * 2.0 ** -10, 2.0 ** -8), (448.0, 448.0), (-0.3, -0.3125),
                                    (76.8, 80.0), (0.0, 0.0), (2.0 ** -9, 2.0 ** -9)])
def test_round_hand_values(x, want):
    assert e4m3_round(np.array([x]))[0] == want


def test_round_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3_round(np.array([470.0]))


def _random_case(rng, B, H, Hkv, N, d):
    # codes of N(0,1) values scaled into the e4m3 range, as a per-tensor quantiser would make
    q8 = _codes_of(rng.standard_normal((B, H, N, d)) * 100)
    k8 = _codes_of(rng.standard_normal((B, Hkv, N, d)) * 100)
    v8 = _codes_of(rng.standard_normal((B, Hkv, N, d)) * 100)
    return q8, k8, v8


@pytest.mark.parametrize("block", [1, 3, 128])
@pytest.mark.parametrize("causal,lens", [(False, None), (True, None), (True, [0, 7, 11]),
                                         (False, [5, 11, 1])])
def test_unrounded_equals_three_pass_definition(block, causal, lens):
    rng = np.random.default_rng(32)
    B, H, Hkv, N, d = 3, 4, 2, 11, 8
    q8, k8, v8 = _random_case(rng, B, H, Hkv, N, d)
    qs, ks, vs, scale = 0.011, 0.007, 0.013, 0.4
    o, lse = attention_fp8_ref(q8, k8, v8, qs, ks, vs, scale, causal=causal, seq_lens=lens,
                               block=block, p_scale=None)
    ro, rl = attention_ref(e4m3_decode(q8) * qs, e4m3_decode(k8) * ks, e4m3_decode(v8) * vs,
                           scale, causal=causal, seq_lens=lens)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_lse_does_not_depend_on_rounding():
    rng = np.random.default_rng(33)
    q8, k8, v8 = _random_case(rng, 1, 2, 2, 300, 16)
    a = attention_fp8_ref(q8, k8, v8, 0.01, 0.01, 0.01, 0.25, causal=True)
    b = attention_fp8_ref(q8, k8, v8, 0.01, 0.01, 0.01, 0.25, causal=True, p_scale=None)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)
    assert not np.allclose(a[0], b[0], rtol=0, atol=1e-9)  # the rounding does act on O


@pytest.mark.parametrize("block", [2, 3, 128])
def test_power_of_two_probabilities_are_exact(block):
    # q = e0 with q_scale = ln 2, keys k_j e0 with integer k_j: every probability relative to
    # any running maximum is 2^(k_j - m), representable after the factor 256 (exponents >= -9).
    ks = np.array([0, -1, -3, 2, -2, 1, -5, 3, 0, -4], dtype=np.float32)
    N = ks.size
    e0 = np.array([1.0, 0.0, 0.0])  # only the first of d = 3 components carries the score
    q8 = _codes_of(np.broadcast_to(e0, (1, 1, N, 3)))
    k8 = _codes_of(ks.reshape(1, 1, N, 1) * e0)
    rng = np.random.default_rng(34)
    v8 = _codes_of(rng.integers(-6, 7, (1, 1, N, 3)).astype(np.float32))
    for causal in (False, True):
        o, lse = attention_fp8_ref(q8, k8, v8, math.log(2.0), 1.0, 0.5, 1.0, causal=causal,
                                   block=block)
        ro, rl = attention_ref(e4m3_decode(q8) * math.log(2.0), e4m3_decode(k8),
                               e4m3_decode(v8) * 0.5, 1.0, causal=causal)
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("block", [1, 2])
def test_two_keys_closed_form(block):
    # scores 0 and ln 0.3: p = (1, 0.3); 64 * 0.3 = 19.2 -> e4m3 20 -> 0.3125
    e0 = np.array([1.0, 0.0, 0.0])
    q8 = _codes_of(np.broadcast_to(e0, (1, 1, 2, 3)))
    k8 = _codes_of(np.array([0.0, 1.0]).reshape(1, 1, 2, 1) * e0)
    v0, v1 = np.array([1.0, -2.0, 0.5]), np.array([3.0, 4.0, -1.5])
    v8 = _codes_of(np.stack([v0, v1]).reshape(1, 1, 2, 3))
    o, lse = attention_fp8_ref(q8, k8, v8, 1.0, math.log(0.3), 1.0, 1.0, block=block)
    np.testing.assert_allclose(o[0, 0, 1], (v0 + 0.3125 * v1) / 1.3, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0, 1], math.log(1.3), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[0, 0, 0], (v0 + 0.3125 * v1) / 1.3, rtol=0, atol=1e-12)


def test_equal_scores_mean_and_causal_row0():
    rng = np.random.default_rng(35)
    N, d = 300, 4
    q8 = _codes_of(np.zeros((1, 1, N, d)))
    k8 = _codes_of(rng.standard_normal((1, 1, N, d)))
    v8 = _codes_of(rng.standard_normal((1, 1, N, d)) * 10)
    v = e4m3_decode(v8)[0, 0] * 0.1
    o, lse = attention_fp8_ref(q8, k8, v8, 1.0, 1.0, 0.1, 0.5)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v.mean(axis=0), (N, d)), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.log(N), rtol=0, atol=1e-12)
    q8 = _codes_of(rng.standard_normal((1, 1, N, d)) * 50)
    o, _ = attention_fp8_ref(q8, k8, v8, 0.02, 1.0, 0.1, 0.5, causal=True)
    np.testing.assert_array_equal(o[0, 0, 0], v[0])


def test_rounding_error_within_e4m3_bound():
    rng = np.random.default_rng(36)
    q8, k8, v8 = _random_case(rng, 1, 2, 1, 400, 16)
    qs, ks, vs, scale = 0.02, 0.02, 0.01, 0.25
    o, _ = attention_fp8_ref(q8, k8, v8, qs, ks, vs, scale, causal=True)
    ro, _ = attention_ref(e4m3_decode(q8) * qs, e4m3_decode(k8) * ks, e4m3_decode(v8) * vs,
                          scale, causal=True)
    # The rounding error of 64 p (p relative to the row's reference m_t <= m) is at most
    # max(2^-4 * 64 p, 2^-10): relative 2^-4 for normals, half the subnormal spacing below.
    # With l >= 1 this bounds |O - O_exact| by 2^-4 sum_j P_ij |V_j| + 2^-16 sum_j |V_j|.
    from oracle import attention_probs_ref
    _, _, p = attention_probs_ref(e4m3_decode(q8) * qs, e4m3_decode(k8) * ks,
                                  e4m3_decode(v8) * vs, scale, causal=True)
    vabs = np.abs(e4m3_decode(v8) * vs)
    floor = 2.0 ** -16 * np.cumsum(vabs[0, 0], axis=0)  # causal row i sees keys 0..i
    for h in range(2):
        bound = 2.0 ** -4 * (p[0, h] @ vabs[0, 0]) + floor + 1e-12
        err = np.abs(o[0, h] - ro[0, h])
        assert (err <= bound).all()
        assert err.max() > 0


@pytest.mark.parametrize("causal,lens", [(False, None), (True, [9, 300])])
def test_row_subset_equals_full(causal, lens):
    rng = np.random.default_rng(37)
    q8, k8, v8 = _random_case(rng, 2, 2, 1, 300, 8)
    full = attention_fp8_ref(q8, k8, v8, 0.01, 0.01, 0.01, 0.3, causal=causal, seq_lens=lens)
    rows = [299, 0, 150, 8, 9]
    sub = attention_fp8_ref(q8, k8, v8, 0.01, 0.01, 0.01, 0.3, causal=causal, seq_lens=lens,
                            rows=rows)
    np.testing.assert_allclose(sub[0], full[0][:, :, rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(sub[1], full[1][:, :, rows], rtol=0, atol=1e-13)


def test_lagging_reference_closed_form():
    # One query, block = 1, scores (log2 units) 0, 1, 1.5, 2.5: the reference is set by key 0
    # and stays there while scores exceed it by at most 2 (p = 1, 2, 2^1.5), then moves to 2.5.
    # Weights before the move: 64 p = 64, 128, 181.02 -> e4m3 64, 128, 176; after it, 64.
    e0 = np.array([1.0, 0.0])
    s2 = np.array([0.0, 1.0, 1.5, 2.5])
    q8 = _codes_of(np.broadcast_to(e0, (1, 1, 4, 2)))
    k8 = _codes_of(s2.reshape(1, 1, 4, 1) * e0)           # 0, 1, 1.5, 2.5 are e4m3 values
    rng = np.random.default_rng(38)
    v = rng.integers(-4, 5, (4, 2)).astype(np.float64)
    v8 = _codes_of(v.reshape(1, 1, 4, 2))
    o, lse = attention_fp8_ref(q8, k8, v8, math.log(2.0), 1.0, 1.0, 1.0, block=1)
    a = 2.0 ** -2.5
    num = a * (1.0 * v[0] + 2.0 * v[1] + 2.75 * v[2]) + 1.0 * v[3]
    den = a * (1.0 + 2.0 + 2.0 ** 1.5) + 1.0
    np.testing.assert_allclose(o[0, 0, 3], num / den, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0, 3], math.log(np.exp2(s2).sum()), rtol=0, atol=1e-12)
    # lag = 0 is the plain running maximum: the reference follows every new maximum
    o0, _ = attention_fp8_ref(q8, k8, v8, math.log(2.0), 1.0, 1.0, 1.0, block=1, lag=0.0)
    w = [2.0 ** -2.5, 2.0 ** -1.5, 2.0 ** -1.0, 1.0]      # each 64 p exact at its own reference
    np.testing.assert_allclose(o0[0, 0, 3], (np.array(w) @ v) / sum(w), rtol=0, atol=1e-12)
