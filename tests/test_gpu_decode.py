"""GPU parity of fa_paged_decode (through the C ABI) against the fp64 oracle."""

import numpy as np
import pytest
import torch

from io_aware_attention_02_amd import fa_paged_decode
from io_aware_attention_02_amd.inputs import WORKLOADS, paged_decode_inputs
from oracle import paged_decode_ref

from gpu_common import TOL_LSE, TOL_O_BF16, device, f64, max_abs, say

pytestmark = pytest.mark.gpu


def _run(q, kc, vc, table, lens, scale=None):
    dev = device()
    o, lse = fa_paged_decode(q.to(dev), kc.to(dev), vc.to(dev), table.to(dev), lens.to(dev),
                             scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _check(q, kc, vc, table, lens, o, lse, scale, seqs=None):
    seqs = range(q.shape[0]) if seqs is None else seqs
    kcf, vcf = kc.float().numpy(), vc.float().numpy()       # exact bf16 -> fp32 upcast
    tb = table.numpy()
    go, gl = f64(o), f64(lse)
    for b in seqs:
        L = int(lens[b])
        ro, rl = paged_decode_ref(f64(q[b:b + 1]), kcf, vcf, tb[b:b + 1], [L], scale)
        if L == 0:
            assert (go[b] == 0).all() and np.isneginf(gl[b]).all(), f"seq {b}: empty sequence fill"
            continue
        eo, el = max_abs(go[b], ro[0]), max_abs(gl[b], rl[0])
        assert eo <= TOL_O_BF16, f"seq {b} (L={L}): O max-abs {eo:.3e}"
        assert el <= TOL_LSE, f"seq {b} (L={L}): LSE max-abs {el:.3e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (16, 1), (32, 8)])
def test_decode_lengths(d, hq, hkv):
    lens = [1, 15, 16, 17, 31, 32, 33, 511, 512, 513, 1000, 1537, 0]
    say(f"fa_paged_decode d={d} Hq={hq} Hkv={hkv} lens={lens}")
    q, kc, vc, table, sl = paged_decode_inputs(len(lens), hq, hkv, d, 16, seed=300 + d + hq,
                                               seq_lens=lens, spare_blocks=5)
    o, lse = _run(q, kc, vc, table, sl)
    _check(q, kc, vc, table, sl, o, lse, 1 / d ** 0.5)


def test_decode_long_and_custom_scale():
    lens = [32768, 4097, 20000]
    say(f"fa_paged_decode long lens={lens}")
    q, kc, vc, table, sl = paged_decode_inputs(len(lens), 32, 8, 128, 16, seed=321, seq_lens=lens)
    for scale in (0.0, 0.2):
        o, lse = _run(q, kc, vc, table, sl, scale=scale)
        _check(q, kc, vc, table, sl, o, lse, scale)


def test_decode_block_relabelling_is_bitwise_invisible():
    say("fa_paged_decode block relabelling")
    lens = [700, 33, 1600]
    q, kc, vc, table, sl = paged_decode_inputs(3, 16, 4, 128, 16, seed=322, seq_lens=lens,
                                               spare_blocks=9)
    o1, l1 = _run(q, kc, vc, table, sl)
    g = torch.Generator().manual_seed(5)
    relabel = torch.randperm(kc.shape[0], generator=g)
    kc2 = torch.empty_like(kc)
    vc2 = torch.empty_like(vc)
    kc2[relabel] = kc
    vc2[relabel] = vc
    table2 = torch.where(table >= 0, relabel[table.clamp(min=0).long()].to(torch.int32), table)
    o2, l2 = _run(q, kc2, vc2, table2, sl)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_nan_in_unused_slots_stays_out():
    say("fa_paged_decode NaN in slots past the length")
    lens = [17, 40, 5]
    q, kc, vc, table, sl = paged_decode_inputs(3, 8, 2, 128, 16, seed=323, seq_lens=lens)
    for b, L in enumerate(lens):
        last = int(table[b, (L - 1) // 16])
        kc[last, L % 16 or 16:] = float("nan")
        vc[last, L % 16 or 16:] = float("nan")
    o, lse = _run(q, kc, vc, table, sl)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    _check(q, kc, vc, table, sl, o, lse, 1 / 128 ** 0.5)


def test_decode_deterministic():
    say("fa_paged_decode determinism")
    q, kc, vc, table, sl = paged_decode_inputs(8, 32, 8, 128, 16, len_lo=1, len_hi=3000, seed=324)
    o1, l1 = _run(q, kc, vc, table, sl)
    o2, l2 = _run(q, kc, vc, table, sl)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("seed,pool", [(None, None), (101, None), (102, None), (103, None),
                                       (None, 4096)])  # the workload's seed, repeats, shared pool
def test_paged_decode_workload(seed, pool):
    w = WORKLOADS["paged_decode"]
    seed = w["seed"] if seed is None else seed
    say(f"fa_paged_decode 64 seqs Hq=32 Hkv=8 d=128 lens U[512,32768] (every sequence), seed {seed}"
        f", pool {pool or 'distinct blocks'}")
    q, kc, vc, table, sl = paged_decode_inputs(w["S"], w["Hq"], w["Hkv"], w["d"], w["block_size"],
                                               w["len_lo"], w["len_hi"], seed=seed, pool_blocks=pool)
    o, lse = _run(q, kc, vc, table, sl)
    _check(q, kc, vc, table, sl, o, lse, 1 / 128 ** 0.5)


@pytest.mark.parametrize("max_blocks", [255, 256, 512])
def test_decode_range_counts_around_the_xcd_padding(max_blocks):
    # 255 blocks = 8 ranges of 512 tokens (raised to 15 per sequence), 256 = 8 (15), 512 = 16
    # (23): sequences of every length up to the table's capacity, empty ones included.  With 40
    # sequences and 4 kv heads the grid is too small for 1024-token ranges (at most 40 * 4 * 8 =
    # 1280 waves, under four rounds of 1280), so this covers the 512-token path; the 1024-token
    # one is tested below.
    S = 40
    lens = [0] + [int(x) for x in np.linspace(1, max_blocks * 16, S - 1)]
    say(f"fa_paged_decode {S} seqs, block table of {max_blocks} blocks, lens 0..{max_blocks * 16}")
    q, kc, vc, table, sl = paged_decode_inputs(S, 16, 4, 128, 16, seed=330 + max_blocks,
                                               seq_lens=lens)
    if table.shape[1] < max_blocks:  # widen the table to the capacity under test (unused: -1)
        pad = torch.full((S, max_blocks - table.shape[1]), -1, dtype=torch.int32)
        table = torch.cat([table, pad], dim=1)
    o, lse = _run(q, kc, vc, table, sl)
    _check(q, kc, vc, table, sl, o, lse, 1 / 128 ** 0.5)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_1024_token_ranges_ragged(d):
    # A block table 2048 blocks wide (32768 tokens) for 64 sequences and 8 kv heads puts
    # 64 * 8 * 32 = 16384 waves in a grid of 1024-token ranges, so the launch takes that range
    # length (it needs a table of more than 7168 tokens and 5120 waves); the
    # lengths sit around its edges (and the 512-token ones), with one empty sequence and one at
    # the table's capacity.  The other sequences stay short so that the cache stays small.
    S = 64
    edge = [0, 1, 15, 16, 17, 511, 512, 513, 1023, 1024, 1025, 2047, 2048, 2049, 3073, 32768]
    lens = edge + [int(x) for x in np.linspace(2, 3000, S - len(edge))]
    say(f"fa_paged_decode d={d} {S} seqs, block table of 2048 blocks, 1024-token ranges, lens {edge} + short")
    q, kc, vc, table, sl = paged_decode_inputs(S, 32, 8, d, 16, seed=360 + d, seq_lens=lens)
    assert table.shape[1] == 2048
    o, lse = _run(q, kc, vc, table, sl)
    _check(q, kc, vc, table, sl, o, lse, 1 / d ** 0.5)


def test_decode_shared_pool_with_repeated_ids():
    # The literal reading of the decode workload's pool: 4096 physical blocks that every
    # sequence draws its ids from, with replacement.
    lens = [1, 17, 500, 4097, 9000, 20000, 32768, 0]
    say(f"fa_paged_decode 4096-block shared pool, ids drawn with replacement, lens={lens}")
    q, kc, vc, table, sl = paged_decode_inputs(len(lens), 32, 8, 128, 16, seed=324, seq_lens=lens,
                                               pool_blocks=4096)
    table[2, 9] = table[2, 4]          # the same block twice in one sequence, for certain
    o, lse = _run(q, kc, vc, table, sl)
    _check(q, kc, vc, table, sl, o, lse, 1 / 128 ** 0.5)


def test_decode_block_ids_outside_the_pool_read_as_zeros():
    # An id outside [0, num_blocks) is never dereferenced: that block's keys and values read as
    # zeros.  The oracle sees the same table with those ids pointing at an all-zero block.
    lens = [700, 33, 1600]
    q, kc, vc, table, sl = paged_decode_inputs(3, 16, 4, 128, 16, seed=325, seq_lens=lens,
                                               spare_blocks=2)
    P = kc.shape[0]
    bad = table.clone()
    bad[0, 5] = P
    bad[1, 1] = -1
    bad[2, 99] = 1 << 30
    o, lse = _run(q, kc, vc, bad, sl)
    kz = torch.cat([kc, torch.zeros_like(kc[:1])])
    vz = torch.cat([vc, torch.zeros_like(vc[:1])])
    ref_table = table.clone()
    ref_table[0, 5] = P
    ref_table[1, 1] = P
    ref_table[2, 99] = P
    _check(q, kz, vz, ref_table, sl, o, lse, 1 / 128 ** 0.5)
