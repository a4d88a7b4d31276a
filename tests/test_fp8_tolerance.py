"""The FP8 tolerance (tests/fp8_bounds.py) separates correct rounding from real mistakes.

CPU only.  A stand-in for the kernel's arithmetic -- ``attention_fp8_ref``, which models one
rounding scheme (online softmax over 64-key blocks, a lagging reference or one fixed after the
first 128 keys, probabilities rounded as e4m3(64 p) / 64), stored to bf16 -- must pass both
checks against the exact attention of the dequantised inputs; so must other blockings of the
same scheme, since the tolerance is derived
from the format and not from one schedule.  Outputs with a plausible mistake (a block of values
lost, values off by one key, the scores against the wrong key head) must fail.
"""

import numpy as np
import pytest
import torch

from io_aware_attention_02_amd.inputs import fp8_inputs
from oracle import attention_fp8_ref, attention_probs_ref, e4m3_decode

from fp8_bounds import check_against_exact

B, H, HKV, N, D = 1, 4, 2, 1024, 128


def case_fn():
    q8, k8, v8, sc, _ = fp8_inputs(B, H, HKV, N, D, seed=31)
    scale = 1 / D ** 0.5
    q = e4m3_decode(q8.numpy()) * sc[0]
    k = e4m3_decode(k8.numpy()) * sc[1]
    v = e4m3_decode(v8.numpy()) * sc[2]
    ro, _, probs = attention_probs_ref(q, k, v, scale)
    return q8, k8, v8, sc, scale, v, ro, probs


@pytest.fixture(scope="module")
def case():
    return case_fn()


def _bf16(x):
    return torch.tensor(x).to(torch.bfloat16).double().numpy()


def _model(case, v8=None, **kw):
    q8, k8, v8_, sc, scale, _, _, _ = case
    v8 = v8_ if v8 is None else v8
    return _bf16(attention_fp8_ref(q8.numpy(), k8.numpy(), v8.numpy(), *sc, scale, **kw)[0])


def _check(case, go):
    *_, v, ro, probs = case
    return check_against_exact(go, ro, probs, v, H // HKV)


@pytest.mark.parametrize("kw", [dict(), dict(lag=0.0), dict(block=128, lag=3.0, p_scale=32.0),
                                dict(block=16), dict(headroom=4.0), dict(headroom=4.0, first=64)],
                         ids=["block64_lag2", "block64_lag0", "block128_lag3", "block16",
                              "fixed_ref_h4", "fixed_ref_h4_first64"])
def test_rounded_probabilities_pass(case, kw):
    worst, agg = _check(case, _model(case, **kw))
    assert worst <= 0.5 and agg <= 0.6, (worst, agg)


def test_a_lost_block_of_values_fails(case):
    v8 = case[2].clone()
    v8[:, :, 320:384] = 0                       # one 64-key block of values lost
    with pytest.raises(AssertionError):
        worst, agg = _check(case, _model(case, v8=v8))
        assert agg <= 1.0, agg


def test_values_off_by_one_key_fail(case):
    v8 = case[2].clone()
    v8[:, :, 1:] = case[2][:, :, :-1]
    with pytest.raises(AssertionError):
        _check(case, _model(case, v8=v8))


def test_wrong_kv_head_fails(case):
    q8, k8, v8, sc, scale, v, ro, probs = case
    wrong = attention_fp8_ref(q8.numpy(), k8.numpy()[:, ::-1].copy(), v8.numpy(), *sc, scale)[0]
    with pytest.raises(AssertionError):
        worst, agg = _check(case, _bf16(wrong))
        assert agg <= 1.0, agg


def test_fixed_reference_falls_back_where_a_late_key_dominates():
    # Row 700 of head 0 gets a key (650) equal to its own query: its score exceeds the first
    # 128 keys' maximum by far more than the fixed reference's 2^4 headroom admits (64 p > 464),
    # so the row is computed with the lagging reference; the other rows keep the fixed one and
    # still round differently from it.
    q8, k8, v8, sc, scale, _, _, _ = case_fn()
    k8 = k8.clone()
    k8[0, 0, 650] = q8[0, 0, 700]
    args = (q8.numpy(), k8.numpy(), v8.numpy(), *sc, scale)
    lagging = attention_fp8_ref(*args)[0]
    fixed = attention_fp8_ref(*args, headroom=4.0)[0]
    assert np.array_equal(fixed[0, 0, 700], lagging[0, 0, 700])
    assert not np.array_equal(fixed[0, 0, 699], lagging[0, 0, 699])
    exact = attention_fp8_ref(*args, p_scale=None)[0]
    assert np.abs(fixed - exact).max() < 0.05


def test_fixed_reference_and_lse_match_the_lagging_one():
    # The LSE uses unrounded probabilities: both references give the exact log-sum-exp.
    q8, k8, v8, sc, scale, _, _, _ = case_fn()
    args = (q8.numpy(), k8.numpy(), v8.numpy(), *sc, scale)
    lse_lag = attention_fp8_ref(*args)[1]
    lse_fix = attention_fp8_ref(*args, headroom=4.0)[1]
    np.testing.assert_allclose(lse_fix, lse_lag, rtol=0, atol=1e-12)
