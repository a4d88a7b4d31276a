"""Seeded generators: same seed gives the same bytes; layouts and ranges are as documented."""

import hashlib

import torch

from io_aware_attention_02_amd.inputs import paged_decode_inputs, prefill_inputs


def _h(*ts):
    m = hashlib.sha256()
    for t in ts:
        m.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return m.hexdigest()


def test_prefill_inputs_are_reproducible():
    a = prefill_inputs(2, 4, 2, 33, 64, "bf16", seed=7, len_lo=5, len_hi=33)
    b = prefill_inputs(2, 4, 2, 33, 64, "bf16", seed=7, len_lo=5, len_hi=33)
    assert _h(*a[:3], a[3]) == _h(*b[:3], b[3])
    c = prefill_inputs(2, 4, 2, 33, 64, "bf16", seed=8)
    assert _h(*a[:3]) != _h(*c[:3])
    q, k, v, lens = a
    assert q.dtype == torch.bfloat16 and q.shape == (2, 4, 33, 64) and k.shape == (2, 2, 33, 64)
    assert lens.dtype == torch.int32 and ((lens >= 5) & (lens <= 33)).all()


def test_bf16_is_round_to_nearest_even_of_float32_draws():
    g = torch.Generator().manual_seed(3)
    ref = torch.randn(1 * 1 * 8 * 64, generator=g, dtype=torch.float32)
    q, _, _, _ = prefill_inputs(1, 1, 1, 8, 64, "bf16", seed=3)
    assert torch.equal(q.reshape(-1), ref.to(torch.bfloat16))


def test_paged_inputs_layout():
    q, kc, vc, table, lens = paged_decode_inputs(5, 8, 2, 64, 16, len_lo=1, len_hi=70, seed=9)
    q2, kc2, vc2, table2, lens2 = paged_decode_inputs(5, 8, 2, 64, 16, len_lo=1, len_hi=70, seed=9)
    assert _h(q, kc, vc, table, lens) == _h(q2, kc2, vc2, table2, lens2)
    nb = [(int(L) + 15) // 16 for L in lens]
    assert kc.shape == (sum(nb), 16, 2, 64) and table.dtype == torch.int32
    used = torch.cat([table[b, :n] for b, n in enumerate(nb)])
    assert sorted(used.tolist()) == list(range(sum(nb)))          # each block used once
    for b, n in enumerate(nb):
        assert (table[b, n:] == -1).all()


def test_paged_inputs_unchanged_by_the_pool_option_default():
    # The default recipe (distinct ids by permutation) draws the same bytes as before the shared
    # pool option existed: the permutation path consumes the generator as it always did.
    g = torch.Generator().manual_seed(9)
    lens = torch.randint(1, 71, (5,), generator=g, dtype=torch.int64)
    nb = [(int(L) + 15) // 16 for L in lens]
    perm = torch.randperm(sum(nb), generator=g, dtype=torch.int64)
    _, _, _, table, _ = paged_decode_inputs(5, 8, 2, 64, 16, len_lo=1, len_hi=70, seed=9)
    assert torch.equal(torch.cat([table[b, :n] for b, n in enumerate(nb)]).long(), perm)


def test_shared_pool_draws_ids_with_replacement():
    from io_aware_attention_02_amd.inputs import paged_prefill_inputs
    q, kc, vc, table, lens = paged_decode_inputs(8, 8, 2, 64, 16, len_lo=300, len_hi=900, seed=4,
                                                 pool_blocks=64)
    assert kc.shape == (64, 16, 2, 64) and vc.shape == kc.shape
    nb = [(int(L) + 15) // 16 for L in lens]
    used = torch.cat([table[b, :n] for b, n in enumerate(nb)])
    assert ((used >= 0) & (used < 64)).all()
    assert used.unique().numel() < used.numel()                      # ids repeat
    assert any(table[b, :n].unique().numel() < n for b, n in enumerate(nb))   # inside a sequence
    for b, n in enumerate(nb):
        assert (table[b, n:] == -1).all()
    out = paged_prefill_inputs(3, 4, 2, 64, 32, len_lo=100, len_hi=200, seed=4, pool_blocks=16)
    assert out[1].shape[0] == 16 and int(out[3].max()) < 16
