"""GPU parity of fa_fwd_fp8 (through the C ABI) against the fp64 oracle.

The oracle is the plain definition: the exact attention, in float64, of the tensors the e4m3
codes stand for (codes decoded and multiplied by their descale factors).  The kernel rounds the
probabilities to e4m3 before the P V product, so its outputs differ from that definition by
rounding errors whose size the e4m3 format fixes; ``tests/fp8_bounds.py`` derives the
tolerance (elementwise, and the mean squared error of each tensor against its variance bound)
and ``tests/test_fp8_tolerance.py`` shows on the CPU that it admits correct rounding schemes
and rejects plausible mistakes.  The LSE uses unrounded probabilities and is compared with the
LSE tolerance.

Inputs are the N(0,1) prefill tensors quantised per tensor to e4m3 (descale amax / 448).
Shapes cover ragged lengths, both masks, grouped heads and d = 64 / 128; padding lengths with
the e4m3 NaN code in every padded row; scale 0; the 4K workload in full; the 16K workloads on
one sampled row of every 128-row query tile of every head (rows drawn per head) plus the tile
edges.
"""

import numpy as np
import pytest
import torch

from io_aware_attention_02_amd import fa_fwd_fp8
from io_aware_attention_02_amd.inputs import WORKLOADS, fp8_inputs
from oracle import attention_probs_ref, e4m3_decode

from fp8_bounds import check_against_exact
from gpu_common import TOL_LSE, device, f64, max_abs, say, tile_rows

pytestmark = pytest.mark.gpu


def _run(q8, k8, v8, scales, causal, seq_lens=None, scale=None):
    dev = device()
    sl = None if seq_lens is None else seq_lens.to(dev)
    o, lse = fa_fwd_fp8(q8.to(dev), k8.to(dev), v8.to(dev), *scales, scale=scale, causal=causal,
                        seq_lens=sl)
    torch.cuda.synchronize()
    return f64(o), f64(lse)


def _dequantised(q8, k8, v8, scales):
    qs, ks, vs = scales
    return (e4m3_decode(q8.numpy()) * qs, e4m3_decode(k8.numpy()) * ks,
            e4m3_decode(v8.numpy()) * vs)


def _check(q8, k8, v8, scales, causal, lens, scale, go, gl, rows=None):
    """Exact-attention parity of the rows ``rows`` (all rows if None) of every (batch, head)."""
    q, k, v = _dequantised(q8, k8, v8, scales)
    ro, rl, p = attention_probs_ref(q, k, v, scale, causal=causal, seq_lens=lens, rows=rows)
    group = q.shape[1] // k.shape[1]
    worst, agg = check_against_exact(go, ro, p, v, group, lens=lens, rows=rows)
    assert agg <= 1.0, f"mean squared error {agg:.3f} x its e4m3 variance bound"
    N = q.shape[2]
    sel = np.arange(N) if rows is None else np.asarray(rows)
    for b in range(q.shape[0]):
        L = N if lens is None else lens[b]
        ok = sel < L
        if ok.any():
            el = max_abs(gl[b][:, ok], rl[b][:, ok])
            assert el <= TOL_LSE, f"batch {b}: LSE max-abs {el:.3e}"
        if (~ok).any():
            assert (go[b][:, ~ok] == 0).all(), f"batch {b}: padding rows of O not zero"
            assert np.isneginf(gl[b][:, ~ok]).all(), f"batch {b}: padding LSE not -inf"
    say(f"  vs exact attention: worst error / e4m3 bound {worst:.3f}, "
        f"mean squared error / variance bound {agg:.3f}")


def _check_sampled(q8, k8, v8, scales, causal, scale, go, gl, tile, seed):
    """One row of every `tile`-row query tile of every head, drawn per head."""
    H, Hkv = q8.shape[1], k8.shape[1]
    group = H // Hkv
    for h in range(H):
        rows = tile_rows(q8.shape[2], tile, h, seed)
        g = h // group
        _check(q8[:, h:h + 1], k8[:, g:g + 1], v8[:, g:g + 1], scales, causal, None, scale,
               go[:, h:h + 1, rows], gl[:, h:h + 1, rows], rows=rows)


SHAPES = [
    # (B, H, Hkv, N, d, causal)
    (1, 1, 1, 1, 128, False),
    (1, 2, 2, 17, 128, True),
    (1, 2, 1, 63, 64, False),
    (2, 2, 2, 64, 128, True),
    (1, 4, 1, 129, 128, False),
    (1, 2, 2, 200, 64, True),
    (1, 8, 2, 300, 128, True),
    (2, 4, 4, 513, 128, False),
    (1, 4, 2, 1000, 64, True),
    (1, 2, 2, 1031, 128, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}H{s[1]}Hkv{s[2]}N{s[3]}d{s[4]}{'c' if s[5] else ''}" for s in SHAPES])
def test_fp8_shapes(shape):
    B, H, Hkv, N, d, causal = shape
    say(f"fa_fwd_fp8 {shape}")
    q8, k8, v8, scales, _ = fp8_inputs(B, H, Hkv, N, d, seed=401 + N)
    go, gl = _run(q8, k8, v8, scales, causal)
    _check(q8, k8, v8, scales, causal, None, 1 / d ** 0.5, go, gl)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_padding_with_nan_codes(causal):
    # Lengths 0, 1, a ragged middle and full; the padded rows of q, k, v hold the e4m3 NaN code.
    B, H, Hkv, N, d = 4, 4, 2, 300, 128
    say(f"fa_fwd_fp8 padding causal={causal}")
    q8, k8, v8, scales, _ = fp8_inputs(B, H, Hkv, N, d, seed=411)
    lens = [0, 1, 129, N]
    clean = [t.clone() for t in (q8, k8, v8)]
    for b, L in enumerate(lens):
        for t in (q8, k8, v8):
            t[b, :, L:] = 0x7F
    go, gl = _run(q8, k8, v8, scales, causal, seq_lens=torch.tensor(lens, dtype=torch.int32))
    _check(*clean, scales, causal, lens, 1 / d ** 0.5, go, gl)


def test_fp8_scale_zero_gives_mean_of_v():
    B, H, N, d = 1, 2, 300, 64
    q8, k8, v8, scales, _ = fp8_inputs(B, H, H, N, d, seed=412)
    go, gl = _run(q8, k8, v8, scales, False, scale=0.0)
    v = e4m3_decode(v8.numpy()) * scales[2]
    assert max_abs(go, np.broadcast_to(v.mean(axis=2, keepdims=True), go.shape)) <= 2.0 ** -8 * 4
    assert max_abs(gl, np.full(gl.shape, np.log(N))) <= TOL_LSE


def test_fp8_workload_4k_full():
    w = WORKLOADS["fp8_4k"]
    say("fa_fwd_fp8 fp8_4k, every row")
    q8, k8, v8, scales, _ = fp8_inputs(w["B"], w["H"], w["Hkv"], w["N"], w["d"], seed=w["seed"])
    go, gl = _run(q8, k8, v8, scales, w["causal"])
    _check(q8, k8, v8, scales, w["causal"], None, 1 / w["d"] ** 0.5, go, gl)


@pytest.mark.parametrize("name", ["fp8_16k", "fp8_16k_causal"])
def test_fp8_workload_16k_every_query_tile(name):
    w = WORKLOADS[name]
    say(f"fa_fwd_fp8 {name}, a row of every 128-row query tile of every head")
    q8, k8, v8, scales, _ = fp8_inputs(w["B"], w["H"], w["Hkv"], w["N"], w["d"], seed=w["seed"])
    go, gl = _run(q8, k8, v8, scales, w["causal"])
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    _check_sampled(q8, k8, v8, scales, w["causal"], 1 / w["d"] ** 0.5, go, gl, 128, w["seed"])
