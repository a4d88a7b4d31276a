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
edges; keys planted to dominate rows far beyond the first tile's maximum, which send the
kernel's workgroups from the fixed-reference pass to the lagging one.
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


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_long_sequence_every_query_tile(causal):
    # 65573 keys (a ragged last tile) in the eight-wave grid; a row of every 256-row query tile.
    B, H, Hkv, N, d = 1, 2, 1, 65573, 128
    say(f"fa_fwd_fp8 N={N} causal={causal}, a row of every 256-row query tile of every head")
    q8, k8, v8, scales, _ = fp8_inputs(B, H, Hkv, N, d, seed=431)
    go, gl = _run(q8, k8, v8, scales, causal)
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    _check_sampled(q8, k8, v8, scales, causal, 1 / d ** 0.5, go, gl, 256, 431)


# The first pass fixes each row's reference 2^4 above the maximum of its first 128 keys; a
# probability above 7.25 (64 p > 464) has no e4m3 code, and the workgroup recomputes with the
# lagging reference.  A key equal to a row's own query scores about |q|^2 / sqrt(d), far above
# the first tile's maximum of random scores.
HEAD_LOG2, P_LIMIT = 4.0, 464.0 / 64.0
FALLBACK = [
    # (B, H, Hkv, N, d, causal, [(head, row, key), ...]); 4-wave (small grid) and 8-wave grids
    (1, 4, 2, 1031, 128, False, [(0, 700, 650), (1, 1000, 300), (2, 1030, 1030), (3, 100, 900)]),
    (1, 4, 2, 1031, 128, True, [(0, 700, 650), (1, 1000, 300), (2, 1030, 1030), (3, 256, 200)]),
    (1, 8, 2, 8192, 128, False, [(0, 5000, 4000), (5, 100, 3000)]),
    (1, 8, 2, 8192, 128, True, [(0, 5000, 4000), (6, 8191, 130)]),
    (1, 4, 2, 1031, 64, False, [(0, 150, 129), (1, 1030, 200), (2, 300, 129), (3, 500, 250)]),
    (1, 4, 2, 1031, 64, True, [(0, 150, 129), (1, 1030, 200), (2, 300, 129), (3, 500, 250)]),
]


@pytest.mark.parametrize("case", FALLBACK,
                         ids=[f"N{c[3]}H{c[1]}d{c[4]}{'c' if c[5] else ''}" for c in FALLBACK])
def test_fp8_fixed_reference_fallback(case):
    B, H, Hkv, N, d, causal, plants = case
    say(f"fa_fwd_fp8 fallback N={N} H={H} causal={causal} plants={plants}")
    q8, k8, v8, scales, _ = fp8_inputs(B, H, Hkv, N, d, seed=421)
    group = H // Hkv
    for h, i, j in plants:
        k8[0, h // group, j] = q8[0, h, i]
    q, k, _ = _dequantised(q8, k8, v8, scales)
    scale = 1 / d ** 0.5
    sl2 = scale / np.log(2.0)
    for h, i, j in plants:  # the planted key outgrows what the fixed reference admits
        s = (q[0, h, i] @ k[0, h // group, : (i + 1 if causal else N)].T) * sl2
        assert s.max() - s[:128].max() > HEAD_LOG2 + np.log2(P_LIMIT) + 1.0, (h, i, j)
    go, gl = _run(q8, k8, v8, scales, causal)
    wg_rows = 256 if B * H * ((N + 255) // 256) >= 256 else 128
    for h in range(H):
        rows = set(tile_rows(N, 128, h, 421))
        for hp, i, _ in plants:  # every row of a planted row's workgroup (all heads of it)
            if hp == h:
                rows.update(range(i - i % wg_rows, min(N, i - i % wg_rows + wg_rows)))
        rows = np.array(sorted(rows))
        g = h // group
        _check(q8[:, h:h + 1], k8[:, g:g + 1], v8[:, g:g + 1], scales, causal, None, scale,
               go[:, h:h + 1, rows], gl[:, h:h + 1, rows], rows=rows)
