"""GPU parity of fa_paged_prefill (through the C ABI) against the fp64 oracle.

Each sequence's newest Q_b tokens attend, causally with the offset L_b - Q_b, to every cached
token gathered through the block table.  Shapes cover chunk lengths 0, 1, a few, a full tile
and the whole sequence, short and long caches, d = 64 and 128, grouped-query heads, and
sequences of very different work (the kernel serves them heaviest first).
"""

import numpy as np
import pytest
import torch

from io_aware_attention_02_amd import (fa_paged_decode, fa_paged_prefill,
                                     fa_paged_prefill_workspace_bytes)
from io_aware_attention_02_amd.inputs import WORKLOADS, paged_prefill_inputs
from oracle import paged_prefill_ref

from gpu_common import TOL_LSE, TOL_O_BF16, device, f64, max_abs, say, tile_rows

pytestmark = pytest.mark.gpu


def _run(q, kc, vc, table, lens, qlens, scale=None):
    dev = device()
    o, lse = fa_paged_prefill(q.to(dev), kc.to(dev), vc.to(dev), table.to(dev), lens.to(dev),
                              qlens.to(dev), scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _check(q, kc, vc, table, lens, qlens, o, lse, scale, seqs=None):
    seqs = range(q.shape[0]) if seqs is None else seqs
    kcf, vcf = kc.float().numpy(), vc.float().numpy()       # exact bf16 -> fp32 upcast
    tb = table.numpy()
    go, gl = f64(o), f64(lse)
    for b in seqs:
        L, Q = int(lens[b]), int(qlens[b])
        ro, rl = paged_prefill_ref(f64(q[b:b + 1]), kcf, vcf, tb[b:b + 1], [L], [Q], scale)
        if Q > 0:
            eo, el = max_abs(go[b][:, :Q], ro[0][:, :Q]), max_abs(gl[b][:, :Q], rl[0][:, :Q])
            assert eo <= TOL_O_BF16, f"seq {b} (L={L}, Q={Q}): O max-abs {eo:.3e}"
            assert el <= TOL_LSE, f"seq {b} (L={L}, Q={Q}): LSE max-abs {el:.3e}"
        assert (go[b][:, Q:] == 0).all(), f"seq {b}: padding rows of O not zero"
        assert np.isneginf(gl[b][:, Q:]).all(), f"seq {b}: padding rows of LSE not -inf"


CASES = [
    # (S, Hq, Hkv, d, max_q, lens, q_lens)
    (3, 4, 2, 128, 70, [1, 100, 1000], [1, 64, 70]),
    (2, 8, 8, 64, 200, [200, 513], [200, 129]),
    (4, 32, 8, 128, 16, [17, 32, 5000, 16], [16, 1, 16, 16]),
    (3, 4, 1, 128, 300, [0, 300, 77], [0, 300, 0]),
    (2, 16, 4, 128, 640, [640, 4097], [640, 512]),
    (1, 2, 2, 64, 1, [33], [1]),
    # At least 256 query rows per head: eight-wave work items (64 rows of 4 heads, 128 of 2 or
    # 256 of 1), with d = 64 and the head layouts of one and two heads per item.
    (2, 8, 8, 64, 260, [300, 5000], [260, 100]),
    (2, 12, 6, 128, 256, [256, 3000], [256, 200]),
    (2, 6, 2, 64, 300, [2000, 310], [290, 300]),
]


@pytest.mark.parametrize("case", CASES, ids=[f"S{c[0]}Hq{c[1]}Hkv{c[2]}d{c[3]}Q{c[4]}" for c in CASES])
def test_paged_prefill_cases(case):
    S, Hq, Hkv, d, Q, lens, qls = case
    say(f"fa_paged_prefill {case}")
    q, kc, vc, table, sl, ql = paged_prefill_inputs(S, Hq, Hkv, d, Q, seed=301 + Q, seq_lens=lens,
                                                    q_lens=qls, spare_blocks=3)
    o, lse = _run(q, kc, vc, table, sl, ql)
    _check(q, kc, vc, table, sl, ql, o, lse, 1 / d ** 0.5)


def test_paged_prefill_nan_outside_the_sequence_stays_out():
    # NaN in cache slots past each length, in unreferenced blocks and in padding query rows.
    S, Hq, Hkv, d, Q = 3, 8, 2, 128, 96
    lens, qls = [70, 130, 33], [70, 96, 20]
    q, kc, vc, table, sl, ql = paged_prefill_inputs(S, Hq, Hkv, d, Q, seed=311, seq_lens=lens,
                                                    q_lens=qls, spare_blocks=4)
    used = set(table[table >= 0].tolist())
    for blk in range(kc.shape[0]):
        if blk not in used:
            kc[blk] = float("nan")
            vc[blk] = float("nan")
    for b, (L, qn) in enumerate(zip(lens, qls)):
        nb = -(-L // 16)
        last = int(table[b, nb - 1])
        kc[last, L - 16 * (nb - 1):] = float("nan")
        vc[last, L - 16 * (nb - 1):] = float("nan")
        q[b, :, qn:] = float("nan")
    o, lse = _run(q, kc, vc, table, sl, ql)
    q0 = torch.nan_to_num(q, nan=0.0)
    kc0, vc0 = torch.nan_to_num(kc, nan=0.0), torch.nan_to_num(vc, nan=0.0)
    _check(q0, kc0, vc0, table, sl, ql, o, lse, 1 / d ** 0.5)


def test_one_token_chunk_matches_decode():
    # Q_b = 1 is one decode step: compare with fa_paged_decode's results (different kernels).
    S, Hq, Hkv, d = 8, 32, 8, 128
    q, kc, vc, table, sl, _ = paged_prefill_inputs(S, Hq, Hkv, d, 1, seed=312, len_lo=1,
                                                   len_hi=3000, q_lens=[1] * S)
    dev = device()
    ql = torch.ones(S, dtype=torch.int32)
    o, lse = _run(q, kc, vc, table, sl, ql)
    od, ld = fa_paged_decode(q[:, :, 0].contiguous().to(dev), kc.to(dev), vc.to(dev),
                             table.to(dev), sl.to(dev))
    torch.cuda.synchronize()
    assert max_abs(f64(o)[:, :, 0], f64(od)) <= TOL_O_BF16
    assert max_abs(f64(lse)[:, :, 0], f64(ld)) <= TOL_LSE


@pytest.mark.timeout(600)
def test_paged_prefill_workload_every_sequence():
    # All 16 sequences (contexts up to 32K, chunks up to 1024): one row of every 32-row block of
    # each chunk (drawn per sequence; every wave of every query tile), the chunk's edges and the
    # first padding rows, against the row-subset oracle.
    w = WORKLOADS["paged_prefill"]
    say("fa_paged_prefill workload, every sequence")
    q, kc, vc, table, sl, ql = paged_prefill_inputs(w["S"], w["Hq"], w["Hkv"], w["d"], w["max_q"],
                                                    w["block_size"], w["len_lo"], w["len_hi"],
                                                    seed=w["seed"])
    o, lse = _run(q, kc, vc, table, sl, ql)
    assert torch.isfinite(o.float()).all()
    _check_rows(q, kc, vc, table, sl, ql, o, lse, 1 / w["d"] ** 0.5, w["seed"])


def _check_rows(q, kc, vc, table, lens, qlens, o, lse, scale, seed):
    kcf, vcf = kc.float().numpy(), vc.float().numpy()
    tb = table.numpy()
    go, gl = f64(o), f64(lse)
    Qmax = q.shape[2]
    for b in range(q.shape[0]):
        L, Q = int(lens[b]), int(qlens[b])
        rows = set(tile_rows(Qmax, 32, b, seed))
        rows |= {r for r in (0, Q - 2, Q - 1, Q, Q + 1, 127, 128) if 0 <= r < Qmax}
        rows = sorted(rows)
        ro, rl = paged_prefill_ref(f64(q[b:b + 1]), kcf, vcf, tb[b:b + 1], [L], [Q], scale,
                                   rows=rows)
        sel = np.asarray(rows) < Q
        g_o, g_l = go[b][:, rows], gl[b][:, rows]
        if sel.any():
            eo = max_abs(g_o[:, sel], ro[0][:, sel])
            el = max_abs(g_l[:, sel], rl[0][:, sel])
            say(f"  seq {b} (L={L}, Q={Q}): O max-abs {eo:.2e}, LSE {el:.2e}")
            assert eo <= TOL_O_BF16, f"seq {b} (L={L}, Q={Q}): O max-abs {eo:.3e}"
            assert el <= TOL_LSE, f"seq {b} (L={L}, Q={Q}): LSE max-abs {el:.3e}"
        assert (g_o[:, ~sel] == 0).all(), f"seq {b}: padding rows of O not zero"
        assert np.isneginf(g_l[:, ~sel]).all(), f"seq {b}: padding rows of LSE not -inf"


def test_paged_prefill_row_maximum_far_above_first_tile():
    # One cached token scores ~50 log2-units above every token of each row's first key tile
    # (positive queries, that token's keys all 4): the paged instantiation must take the exact
    # fallback pass, re-gathering its blocks through the table.
    S, Hq, Hkv, d, Q = 2, 8, 2, 128, 200
    lens, qls = [3000, 900], [200, 150]
    say("fa_paged_prefill row maximum far above the first tile")
    q, kc, vc, table, sl, ql = paged_prefill_inputs(S, Hq, Hkv, d, Q, seed=312, seq_lens=lens,
                                                    q_lens=qls)
    q = q.abs()
    for b, t in ((0, 1700), (1, 500)):  # tokens before each chunk, visible to all its rows
        kc[int(table[b, t // 16]), t % 16] = 4.0
    o, lse = _run(q, kc, vc, table, sl, ql)
    _check(q, kc, vc, table, sl, ql, o, lse, 1 / d ** 0.5)


# Shared pool: the literal reading of a pool of 4096 physical blocks that every sequence draws
# its ids from, with replacement -- ids repeat across sequences and inside one sequence.
def test_paged_prefill_shared_pool_with_repeated_ids():
    S, Hq, Hkv, d, Q = 4, 32, 8, 128, 300
    lens, qls = [3000, 1200, 640, 5000], [300, 129, 64, 1]
    say("fa_paged_prefill, 4096-block shared pool, ids drawn with replacement")
    q, kc, vc, table, sl, ql = paged_prefill_inputs(S, Hq, Hkv, d, Q, seed=313, seq_lens=lens,
                                                    q_lens=qls, pool_blocks=4096)
    table[0, 7] = table[0, 3]          # the same block twice in one sequence, for certain
    o, lse = _run(q, kc, vc, table, sl, ql)
    _check(q, kc, vc, table, sl, ql, o, lse, 1 / d ** 0.5)


def test_paged_prefill_block_ids_outside_the_pool_read_as_zeros():
    # An id outside [0, num_blocks) is never dereferenced: that block's keys and values read as
    # zeros.  The oracle sees the same table with those ids pointing at an all-zero block.
    S, Hq, Hkv, d, Q = 2, 8, 2, 128, 100
    lens, qls = [700, 300], [100, 40]
    q, kc, vc, table, sl, ql = paged_prefill_inputs(S, Hq, Hkv, d, Q, seed=314, seq_lens=lens,
                                                    q_lens=qls, spare_blocks=2)
    P = kc.shape[0]
    bad = table.clone()
    bad[0, 5] = P                      # one past the pool
    bad[1, 2] = -7                     # negative
    o, lse = _run(q, kc, vc, bad, sl, ql)
    kz = torch.cat([kc, torch.zeros_like(kc[:1])])
    vz = torch.cat([vc, torch.zeros_like(vc[:1])])
    ref_table = table.clone()
    ref_table[0, 5] = P
    ref_table[1, 2] = P
    _check(q, kz, vz, ref_table, sl, ql, o, lse, 1 / d ** 0.5)


# Split key ranges.  With little total work the split length is its minimum, 16 key tiles (1024
# keys), so every query block that sees more keys is cut into pieces whose partial results are
# merged.  The cases cover the head layouts of a work item: 4 query heads per item (group 4 and
# 8, the latter two head subsets per kv head), 2 (group 2), 1 (groups 1 and 3), with four-wave
# items (fewer than 256 query rows per head) and eight-wave ones.
SPLIT_CASES = [
    # (S, Hq, Hkv, d, max_q, lens, q_lens)
    (3, 32, 8, 128, 48, [9000, 4100, 1025], [40, 1, 48]),
    (2, 16, 8, 128, 100, [6000, 2500], [100, 65]),
    (2, 12, 4, 64, 70, [5000, 3000], [70, 33]),
    (2, 8, 8, 128, 40, [7000, 1100], [40, 7]),
    (1, 64, 8, 128, 20, [12000], [20]),
    (2, 4, 1, 64, 130, [2100, 16], [130, 16]),
    # Eight-wave items (at least 256 query rows per head): 1, 2 and 4 heads per item.
    (2, 8, 8, 64, 256, [6000, 2500], [256, 65]),
    (2, 12, 6, 128, 300, [5000, 3000], [300, 33]),
    (1, 32, 8, 64, 256, [9000], [256]),
]

HDR_MERGE, HDR_T = 24, 25  # plan header fields (ints at the start of the workspace)


def _run_ws(q, kc, vc, table, lens, qlens, ws):
    # Outputs start as NaN, so a row the kernels never write fails the comparison.
    dev = device()
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    fa_paged_prefill(q.to(dev), kc.to(dev), vc.to(dev), table.to(dev), lens.to(dev),
                     qlens.to(dev), o=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    hdr = ws[:256].view(torch.int32).cpu()
    return o, lse, int(hdr[HDR_MERGE]), int(hdr[HDR_T])


def _workspace(q, table, Hkv):
    S, Hq, Qmax, d = q.shape
    n = fa_paged_prefill_workspace_bytes(S, Qmax, Hq, Hkv, d, table.shape[1])
    return torch.empty(n, dtype=torch.uint8, device=device())


@pytest.mark.parametrize("case", SPLIT_CASES,
                         ids=[f"S{c[0]}Hq{c[1]}Hkv{c[2]}d{c[3]}Q{c[4]}" for c in SPLIT_CASES])
def test_paged_prefill_split_key_ranges(case):
    S, Hq, Hkv, d, Q, lens, qls = case
    say(f"fa_paged_prefill split {case}")
    q, kc, vc, table, sl, ql = paged_prefill_inputs(S, Hq, Hkv, d, Q, seed=321 + Q, seq_lens=lens,
                                                    q_lens=qls, spare_blocks=2)
    ws = _workspace(q, table, Hkv)
    o, lse, n_merge, T = _run_ws(q, kc, vc, table, sl, ql, ws)
    say(f"  split length {T} tiles, {n_merge} split query blocks")
    assert T == 16 and n_merge > 0
    _check(q, kc, vc, table, sl, ql, o, lse, 1 / d ** 0.5)


def test_paged_prefill_workspace_reuse_is_deterministic():
    # Two different calls through one workspace, then the first again: results are bitwise those
    # of a fresh workspace (the plan rewrites everything it reads; the item order is dynamic but
    # each item's arithmetic and the merge order are fixed).
    S, Hq, Hkv, d, Q = 3, 32, 8, 128, 64
    a = paged_prefill_inputs(S, Hq, Hkv, d, Q, seed=331, seq_lens=[8000, 3000, 1500],
                             q_lens=[64, 9, 40])
    b = paged_prefill_inputs(S, Hq, Hkv, d, Q, seed=332, seq_lens=[700, 5000, 2000],
                             q_lens=[64, 64, 1])
    ws = _workspace(a[0], a[3], Hkv)
    oa1, la1, ma, _ = _run_ws(*a, ws)
    ob, lb, mb, _ = _run_ws(*b, ws)
    oa2, la2, _, _ = _run_ws(*a, ws)
    assert ma > 0 and mb > 0
    ob_fresh, lb_fresh, _, _ = _run_ws(*b, _workspace(b[0], b[3], Hkv))
    assert torch.equal(oa1, oa2) and torch.equal(la1, la2)
    assert torch.equal(ob, ob_fresh) and torch.equal(lb, lb_fresh)
    _check(*a, oa1, la1, 1 / d ** 0.5)
    _check(*b, ob, lb, 1 / d ** 0.5)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cap", [128, 48])
def test_paged_prefill_workload_short_chunks_every_sequence(cap):
    # The 16 workload contexts (up to 32K keys) with every chunk cut to at most `cap` tokens: the
    # long key loops are split (split length 117 and 63 tiles) and merged.
    w = WORKLOADS["paged_prefill"]
    say(f"fa_paged_prefill workload contexts, chunks <= {cap}, every sequence")
    q, kc, vc, table, sl, ql = paged_prefill_inputs(w["S"], w["Hq"], w["Hkv"], w["d"], w["max_q"],
                                                    w["block_size"], w["len_lo"], w["len_hi"],
                                                    seed=w["seed"])
    ql = torch.clamp(ql, max=cap)
    ws = _workspace(q, table, w["Hkv"])
    o, lse, n_merge, T = _run_ws(q, kc, vc, table, sl, ql, ws)
    say(f"  split length {T} tiles, {n_merge} split query blocks")
    assert n_merge > 0
    _check_rows(q, kc, vc, table, sl, ql, o, lse, 1 / w["d"] ** 0.5, w["seed"] + cap)


def test_paged_prefill_more_sequences_than_the_ranked_plan_holds():
    # 600 sequences: past the 512 the plan ranks, so its per-sequence arrays live in the
    # workspace instead of LDS and the natural order is kept.  Short contexts and chunks keep the
    # oracle cheap; every row of every sequence is compared, outputs start as NaN.
    S, Hq, Hkv, d, Q = 600, 4, 1, 64, 16
    g = torch.Generator().manual_seed(341)
    lens = torch.randint(1, 201, (S,), generator=g).tolist()
    qls = [int(torch.randint(1, min(Q, L) + 1, (1,), generator=g)) for L in lens]
    qls[0], lens[1], qls[1] = 0, 16, 16  # an empty chunk and a chunk that is the whole sequence
    say(f"fa_paged_prefill S={S}")
    q, kc, vc, table, sl, ql = paged_prefill_inputs(S, Hq, Hkv, d, Q, seed=341, seq_lens=lens,
                                                    q_lens=qls)
    ws = _workspace(q, table, Hkv)
    o, lse, _, _ = _run_ws(q, kc, vc, table, sl, ql, ws)
    _check(q, kc, vc, table, sl, ql, o, lse, 1 / d ** 0.5)
