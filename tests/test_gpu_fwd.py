"""GPU parity of fa_fwd (through the C ABI) against the fp64 oracle.

Small and ragged shapes are compared element by element; the full-size workloads are run in
the launch configuration the bench times and compared on sampled query rows (the oracle's
definition is row-wise, so a row subset is exact).
"""

import numpy as np
import pytest
import torch

from io_aware_attention_02_amd import fa_fwd
from io_aware_attention_02_amd.inputs import WORKLOADS, prefill_inputs
from oracle import attention_ref

from gpu_common import TOL_LSE, TOL_O_BF16, TOL_O_F32, device, f64, max_abs, say, tile_rows

pytestmark = pytest.mark.gpu


def _run(q, k, v, causal, seq_lens=None, scale=None, dev=None):
    dev = dev or device()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    sl = None if seq_lens is None else seq_lens.to(dev)
    o, lse = fa_fwd(qd, kd, vd, scale=scale, causal=causal, seq_lens=sl)
    torch.cuda.synchronize()
    return o, lse


def _check(q, k, v, o, lse, causal, seq_lens, scale, tol_o, rows=None):
    lens = None if seq_lens is None else seq_lens.tolist()
    ro, rl = attention_ref(f64(q), f64(k), f64(v), scale, causal=causal, seq_lens=lens, rows=rows)
    go, gl = f64(o), f64(lse)
    if rows is not None:
        go, gl = go[:, :, rows], gl[:, :, rows]
    B, H, n = rl.shape
    N = q.shape[2]
    rows_idx = np.arange(N) if rows is None else np.asarray(rows)
    for b in range(B):
        L = N if lens is None else lens[b]
        valid = rows_idx < L
        if valid.any():
            eo = max_abs(go[b][:, valid], ro[b][:, valid])
            el = max_abs(gl[b][:, valid], rl[b][:, valid])
            assert eo <= tol_o, f"batch {b}: O max-abs {eo:.3e} > {tol_o}"
            assert el <= TOL_LSE, f"batch {b}: LSE max-abs {el:.3e} > {TOL_LSE}"
        if (~valid).any():
            assert (go[b][:, ~valid] == 0).all(), f"batch {b}: padded rows of O not zero"
            assert np.isneginf(gl[b][:, ~valid]).all(), f"batch {b}: padded LSE not -inf"


SHAPES = [
    # (B, H, Hkv, N, d, causal)
    (1, 1, 1, 1, 128, False),
    (1, 2, 2, 17, 128, True),
    (1, 2, 1, 63, 64, False),
    (2, 2, 2, 64, 128, True),
    (1, 4, 1, 65, 128, False),
    (1, 2, 2, 127, 64, True),
    (1, 8, 2, 129, 128, True),
    (2, 4, 4, 1000, 128, False),
    (1, 4, 1, 1000, 64, True),
    (1, 2, 2, 4097, 128, True),
    (1, 2, 1, 4097, 64, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}H{s[1]}Hkv{s[2]}N{s[3]}d{s[4]}{'c' if s[5] else ''}" for s in SHAPES])
def test_bf16_shapes(shape):
    B, H, Hkv, N, d, causal = shape
    say(f"fa_fwd bf16 {shape}")
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, "bf16", seed=101 + N)
    o, lse = _run(q, k, v, causal)
    _check(q, k, v, o, lse, causal, None, 1 / d ** 0.5, TOL_O_BF16)


F32_SHAPES = [(1, 1, 1, 1, 64, False), (1, 2, 1, 65, 128, True), (2, 2, 2, 300, 64, True),
              (1, 4, 2, 257, 128, False)]


@pytest.mark.parametrize("shape", F32_SHAPES, ids=[f"B{s[0]}H{s[1]}Hkv{s[2]}N{s[3]}d{s[4]}{'c' if s[5] else ''}" for s in F32_SHAPES])
def test_f32_shapes(shape):
    B, H, Hkv, N, d, causal = shape
    say(f"fa_fwd f32 {shape}")
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, "f32", seed=201 + N)
    o, lse = _run(q, k, v, causal)
    _check(q, k, v, o, lse, causal, None, 1 / d ** 0.5, TOL_O_F32)


@pytest.mark.parametrize("seed", [1, 101, 102, 103])
def test_single_head_fp32_workload(seed):
    w = WORKLOADS["single_head_fp32"]
    say(f"fa_fwd single-head fp32 workload seed {seed}")
    q, k, v, _ = prefill_inputs(w["B"], w["H"], w["Hkv"], w["N"], w["d"], "f32", seed=seed)
    o, lse = _run(q, k, v, False)
    _check(q, k, v, o, lse, False, None, 1 / 8, TOL_O_F32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_padding_mask(dtype, causal):
    say(f"fa_fwd padding {dtype} causal={causal}")
    B, H, Hkv, N, d = 4, 4, 2, 300, 128
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, dtype, seed=7)
    lens = torch.tensor([300, 1, 129, 0], dtype=torch.int32)
    o, lse = _run(q, k, v, causal, lens)
    _check(q, k, v, o, lse, causal, lens, 1 / d ** 0.5,
           TOL_O_BF16 if dtype == "bf16" else TOL_O_F32)


def test_nan_poisoned_padding_stays_out():
    say("fa_fwd NaN-poisoned padding")
    B, H, Hkv, N, d = 2, 4, 1, 260, 128
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, "bf16", seed=8)
    lens = torch.tensor([200, 77], dtype=torch.int32)
    for b, L in enumerate(lens.tolist()):
        q[b, :, L:] = float("nan")
        k[b, :, L:] = float("nan")
        v[b, :, L:] = float("nan")
    for causal in (False, True):
        o, lse = _run(q, k, v, causal, lens)
        _check(q, k, v, o, lse, causal, lens, 1 / d ** 0.5, TOL_O_BF16)


def test_scale_zero_and_custom_scale():
    say("fa_fwd scale 0 and 0.3")
    q, k, v, _ = prefill_inputs(1, 2, 2, 150, 64, "bf16", seed=9)
    for scale in (0.0, 0.3):
        for causal in (False, True):
            o, lse = _run(q, k, v, causal, scale=scale)
            _check(q, k, v, o, lse, causal, None, scale, TOL_O_BF16)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("big_key", [500, 520])
def test_row_maximum_far_above_first_tile(causal, big_key):
    # One key of a later tile scores ~50 log2-units above every key of the first tile for every
    # query row (positive queries, a key of all 4s).  A pass that keeps the first tile's maximum
    # as the reference must notice and redo the rows exactly with the rescaling recurrence.
    # Small grids split each workgroup's keys over two groups of waves (odd and even 64-key
    # tiles): key 500 lies in an odd tile, key 520 in an even one.
    say(f"fa_fwd row maximum far above the first tile causal={causal} key={big_key}")
    B, H, Hkv, N, d = 1, 2, 1, 1000, 128
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, "bf16", seed=12)
    q = q.abs()
    k[:, :, big_key] = 4.0
    o, lse = _run(q, k, v, causal)
    _check(q, k, v, o, lse, causal, None, 1 / d ** 0.5, TOL_O_BF16)


# Grids with at least one 256-row workgroup per CU run the eight-wave kernel; these shapes
# reach it with ragged lengths, grouped heads, padding and the fallback pass.
WIDE = [
    # (B, H, Hkv, N, d, causal, lens)
    (2, 32, 8, 1000, 128, True, [1000, 517]),
    (2, 32, 32, 777, 128, False, [777, 1]),
    (4, 16, 4, 1025, 64, True, [1025, 300, 0, 256]),
]


@pytest.mark.parametrize("shape", WIDE, ids=[f"B{s[0]}H{s[1]}Hkv{s[2]}N{s[3]}d{s[4]}{'c' if s[5] else ''}" for s in WIDE])
def test_wide_grid_shapes(shape):
    B, H, Hkv, N, d, causal, lens = shape
    say(f"fa_fwd wide grid {shape}")
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, "bf16", seed=13 + N)
    sl = torch.tensor(lens, dtype=torch.int32)
    o, lse = _run(q, k, v, causal, sl)
    _check(q, k, v, o, lse, causal, sl, 1 / d ** 0.5, TOL_O_BF16)


# Grids between the two (fewer than one 256-row workgroup per CU, more 128-row workgroups than
# CUs) run four-wave 128-row workgroups, two per CU.
MID = [
    # (B, H, Hkv, N, d, causal, lens)
    (1, 8, 2, 5000, 128, True, [5000]),
    (2, 4, 4, 4500, 64, False, [4500, 2100]),
]


@pytest.mark.parametrize("shape", MID, ids=[f"B{s[0]}H{s[1]}Hkv{s[2]}N{s[3]}d{s[4]}{'c' if s[5] else ''}" for s in MID])
def test_mid_grid_shapes(shape):
    B, H, Hkv, N, d, causal, lens = shape
    say(f"fa_fwd mid grid {shape}")
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, "bf16", seed=15 + N)
    sl = torch.tensor(lens, dtype=torch.int32)
    o, lse = _run(q, k, v, causal, sl)
    _check(q, k, v, o, lse, causal, sl, 1 / d ** 0.5, TOL_O_BF16)


def test_mid_grid_row_maximum_far_above_first_tile():
    # The four-wave 128-row kernel (two workgroups per CU) with per-sequence lengths takes the
    # exact fallback pass too; the big key is visible to the longer sequence only.
    say("fa_fwd mid grid, row maximum far above the first tile")
    B, H, Hkv, N, d = 2, 4, 2, 4600, 128
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, "bf16", seed=16)
    q = q.abs()
    k[:, :, 3000] = 4.0
    sl = torch.tensor([4600, 2500], dtype=torch.int32)
    for causal in (False, True):
        o, lse = _run(q, k, v, causal, sl)
        _check(q, k, v, o, lse, causal, sl, 1 / d ** 0.5, TOL_O_BF16)


def test_wide_grid_row_maximum_far_above_first_tile():
    say("fa_fwd wide grid, row maximum far above the first tile")
    B, H, Hkv, N, d = 2, 32, 8, 1000, 128
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, "bf16", seed=14)
    q = q.abs()
    k[:, :, 700] = 4.0
    o, lse = _run(q, k, v, True)
    _check(q, k, v, o, lse, True, None, 1 / d ** 0.5, TOL_O_BF16)


def test_gqa_equals_repeated_kv_bitwise():
    say("fa_fwd GQA vs repeated-KV MHA")
    B, H, Hkv, N, d = 2, 8, 2, 333, 128
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, "bf16", seed=10)
    lens = torch.tensor([333, 190], dtype=torch.int32)
    o1, l1 = _run(q, k, v, True, lens)
    kr = torch.repeat_interleave(k, H // Hkv, dim=1).contiguous()
    vr = torch.repeat_interleave(v, H // Hkv, dim=1).contiguous()
    o2, l2 = _run(q, kr, vr, True, lens)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_launch_shape_is_invisible(causal, d):
    # The grid size picks the workgroup shape: 24 heads of 2048 rows run 128-row workgroups of
    # four waves, 64 heads run 256-row workgroups of eight.  Both visit each row's keys in the
    # same tiles and order, so the first 24 heads must come out bitwise the same either way: a
    # head or a query tile mapped to the wrong data in one of the two launches shows up here.
    say(f"fa_fwd 24 heads (four-wave) vs 64 heads (eight-wave), d={d}, causal={causal}")
    N = 2048
    q, k, v, _ = prefill_inputs(1, 64, 64, N, d, "bf16", seed=21)
    o64, l64 = _run(q, k, v, causal)
    o24, l24 = _run(q[:, :24].contiguous(), k[:, :24].contiguous(), v[:, :24].contiguous(), causal)
    assert torch.equal(o24, o64[:, :24]) and torch.equal(l24, l64[:, :24])
    _check(q[:, :2], k[:, :2], v[:, :2], o24[:, :2], l24[:, :2], causal, None, 1 / d ** 0.5,
           TOL_O_BF16, rows=tile_rows(N, 128, head=0))


def test_deterministic():
    say("fa_fwd determinism")
    q, k, v, _ = prefill_inputs(1, 4, 4, 2048, 128, "bf16", seed=11)
    o1, l1 = _run(q, k, v, False)
    o2, l2 = _run(q, k, v, False)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("seed", [None, 101, 102, 103])  # the workload's own seed, then repeats
def test_prefill_4k_workload_full(seed):
    w = WORKLOADS["prefill_4k"]
    seed = w["seed"] if seed is None else seed
    say(f"fa_fwd B=1 H=8 N=4096 d=128 bf16, every row, seed {seed}")
    q, k, v, _ = prefill_inputs(w["B"], w["H"], w["Hkv"], w["N"], w["d"], "bf16", seed=seed)
    o, lse = _run(q, k, v, False)
    _check(q, k, v, o, lse, False, None, 1 / 128 ** 0.5, TOL_O_BF16)


def _check_every_tile(q, k, v, o, lse, causal, seq_lens, scale, tile, seed):
    """One row of every `tile`-row query tile of every (batch, head), drawn per head, plus the
    tile edges and, with per-sequence lengths, the rows around each length (padding fill
    included)."""
    B, H, N = q.shape[0], q.shape[1], q.shape[2]
    group = H // k.shape[1]
    for b in range(B):
        for h in range(H):
            rows = set(tile_rows(N, tile, h + H * b, seed))
            if seq_lens is not None:
                L = int(seq_lens[b])
                rows |= {r for r in (L - 2, L - 1, L, L + 1) if 0 <= r < N}
            rows = sorted(rows)
            g = h // group
            sl = None if seq_lens is None else seq_lens[b:b + 1]
            _check(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                   o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], causal, sl, scale, TOL_O_BF16,
                   rows=rows)


@pytest.mark.parametrize("name", ["prefill_16k", "prefill_16k_causal"])
def test_prefill_16k_workload_every_query_tile(name):
    w = WORKLOADS[name]
    say(f"fa_fwd {name}: a row of every 256-row query tile of every head")
    q, k, v, _ = prefill_inputs(w["B"], w["H"], w["Hkv"], w["N"], w["d"], "bf16", seed=w["seed"])
    o, lse = _run(q, k, v, w["causal"])
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    _check_every_tile(q, k, v, o.cpu(), lse.cpu(), w["causal"], None, 1 / 128 ** 0.5, 256, w["seed"])


# Causal grids that one or two rounds of 256-row tiles would leave to their heaviest tile run
# 128-row tiles in pairs (i, n - 1 - i): N = 8192 (64 tiles per head), N = 8000 (63: the middle
# tile alone), grouped heads with a ragged and a full length (padding tiles inside pairs), d = 64.
PAIRED = [
    # (B, H, Hkv, N, d, lengths)
    (1, 8, 8, 8192, 128, None),
    (1, 8, 8, 8000, 128, None),
    (2, 8, 2, 4096, 128, [4096, 2500]),
    (1, 8, 8, 8192, 64, None),
]


def _paired_launch(B, H, N):
    # The launcher's rule (fa_fwd_bf16.hip): 256-row tiles would give one or two rounds over the
    # 256 CUs, and the pairs of 128-row tiles still give every CU a workgroup.
    wide = B * H * -(-N // 256)
    pairs = B * H * ((-(-N // 128) + 1) // 2)
    return 256 <= wide < 512 and pairs >= 256


@pytest.mark.parametrize("case", PAIRED, ids=[f"B{c[0]}H{c[1]}Hkv{c[2]}N{c[3]}d{c[4]}" for c in PAIRED])
def test_causal_paired_query_tiles(case):
    B, H, Hkv, N, d, lens = case
    assert _paired_launch(B, H, N)
    say(f"fa_fwd causal paired tiles {case}: a row of every 128-row query tile of every head")
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, "bf16", seed=41)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32)
    o, lse = _run(q, k, v, True, seq_lens=sl)
    _check_every_tile(q, k, v, o.cpu(), lse.cpu(), True, sl, 1 / d ** 0.5, 128, 41)


@pytest.mark.parametrize("causal", [False, True])
def test_long_sequence_every_query_tile(causal):
    # 65573 keys (1025 key tiles, a ragged last one): the eight-wave grid over long rows.
    B, H, Hkv, N, d = 1, 2, 1, 65573, 128
    say(f"fa_fwd N={N} causal={causal}: a row of every 256-row query tile of every head")
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, "bf16", seed=31)
    o, lse = _run(q, k, v, causal)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    _check_every_tile(q, k, v, o.cpu(), lse.cpu(), causal, None, 1 / d ** 0.5, 256, 31)


def test_gqa_varlen_workload_every_query_tile():
    w = WORKLOADS["gqa_varlen_8k"]
    say("fa_fwd GQA causal varlen B=4 H=32 Hkv=8 N=8192: a row of every 256-row tile of every head")
    q, k, v, lens = prefill_inputs(w["B"], w["H"], w["Hkv"], w["N"], w["d"], "bf16", seed=w["seed"],
                                   len_lo=w["len_lo"], len_hi=w["len_hi"])
    o, lse = _run(q, k, v, True, lens)
    _check_every_tile(q, k, v, o.cpu(), lse.cpu(), True, lens, 1 / 128 ** 0.5, 256, w["seed"])
