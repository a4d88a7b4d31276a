"""Seeded synthetic inputs shared by the kernels' tests, the bench and the oracle checks.

This module only draws random numbers and lays them out; it holds none of attention's
arithmetic, so both the HIP path and the CPU oracle can consume its output without sharing
code.  Every tensor is drawn on the CPU from a ``torch.Generator`` seeded explicitly, so a
given (shape, seed) always yields the same bytes on any host.

Recipe (the workload list that the measurements quote):
* prefill: q, k, v drawn in that order as float32 N(0, 1), then rounded to the storage dtype
  (bf16 round-to-nearest-even, or kept float32); layout [B, H, N, d] / [B, Hkv, N, d].
  With per-sequence lengths, ``seq_lens`` is drawn after v, uniform in [lo, hi].
* chunked prefill against the paged cache: the decode recipe for the lengths, the block
  placement and the pools, except that q is [S, Hq, Qmax, d]; the chunk lengths q_lens are
  drawn last, uniform in [1, min(Qmax, L_b)] (0 for an empty sequence), unless given.
* backward: the output gradient dO [B, H, N, d] is drawn from its own generator (seed + 1000)
  as float32 N(0, 1) rounded to the storage dtype.
* paged decode: ``seq_lens`` uniform in [lo, hi] first, then a random permutation that places
  each sequence's logical blocks in the pool, then q [S, Hq, d], then the K pool and the V pool
  [num_blocks, block_size, Hkv, d], all N(0, 1) rounded to bf16.  Unused block-table entries
  are -1.  The pool holds exactly sum(ceil(L_b / block_size)) blocks, so every cached byte is
  distinct and comes from HBM once per decode step.
* shared fixed pool (``pool_blocks=P``): the literal reading of a pool of P physical blocks
  that every sequence draws from.  Instead of the permutation, each logical block's id is drawn
  uniformly from [0, P) with replacement, so ids repeat across sequences and inside one
  sequence; the pools then hold P blocks.  The rest of the recipe is unchanged.
"""

import math

import torch

__all__ = [
    "prefill_inputs",
    "output_gradient",
    "paged_prefill_inputs",
    "varlen_lengths",
    "paged_decode_inputs",
    "WORKLOADS",
    "fp8_inputs",
]

# The five workloads the measurements and parity cases are quoted on.
WORKLOADS = {
    "single_head_fp32": dict(B=1, H=1, Hkv=1, N=256, d=64, dtype="f32", causal=False, seed=1),
    "prefill_4k": dict(B=1, H=8, Hkv=8, N=4096, d=128, dtype="bf16", causal=False, seed=2),
    "prefill_16k": dict(B=1, H=8, Hkv=8, N=16384, d=128, dtype="bf16", causal=False, seed=3),
    "prefill_16k_causal": dict(B=1, H=8, Hkv=8, N=16384, d=128, dtype="bf16", causal=True, seed=3),
    "gqa_varlen_8k": dict(B=4, H=32, Hkv=8, N=8192, d=128, dtype="bf16", causal=True, seed=4,
                          len_lo=2048, len_hi=8192),
    "paged_decode": dict(S=64, Hq=32, Hkv=8, d=128, block_size=16, len_lo=512, len_hi=32768,
                         seed=5),
    # FP8 forward: the 16K prefill shapes with e4m3 inputs (per-tensor scales)
    "fp8_16k": dict(B=1, H=8, Hkv=8, N=16384, d=128, causal=False, seed=7),
    "fp8_16k_causal": dict(B=1, H=8, Hkv=8, N=16384, d=128, causal=True, seed=7),
    "fp8_4k": dict(B=1, H=8, Hkv=8, N=4096, d=128, causal=False, seed=8),
    # chunked prefill against the paged cache: chunks of up to 1024 new tokens
    "paged_prefill": dict(S=16, Hq=32, Hkv=8, d=128, max_q=1024, block_size=16, len_lo=1024,
                          len_hi=32768, seed=6),
}

_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _randn(shape, gen, dtype, chunk=1 << 26):
    """N(0,1) float32 draws rounded to ``dtype``; drawn in chunks to bound host memory."""
    out = torch.empty(shape, dtype=dtype)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        flat[s:e] = torch.randn(e - s, generator=gen, dtype=torch.float32).to(dtype)
    return out


def prefill_inputs(B, H, Hkv, N, d, dtype="bf16", seed=0, len_lo=None, len_hi=None):
    """(q, k, v, seq_lens) on the CPU.  seq_lens is None unless len_lo/len_hi are given."""
    dt = _DTYPES[dtype]
    g = _gen(seed)
    q = _randn((B, H, N, d), g, dt)
    k = _randn((B, Hkv, N, d), g, dt)
    v = _randn((B, Hkv, N, d), g, dt)
    seq_lens = None
    if len_lo is not None:
        seq_lens = varlen_lengths(B, len_lo, len_hi, g)
    return q, k, v, seq_lens


def fp8_inputs(B, H, Hkv, N, d, seed=0, len_lo=None, len_hi=None):
    """(q8, k8, v8, (q_scale, k_scale, v_scale), seq_lens) on the CPU.

    The bf16 N(0,1) tensors of ``prefill_inputs`` quantised per tensor the usual way: descale
    factor amax / 448 (the largest e4m3 value), codes = the tensor divided by it, rounded to
    e4m3 by torch's float8_e4m3fn cast and returned as uint8.
    """
    q, k, v, seq_lens = prefill_inputs(B, H, Hkv, N, d, "bf16", seed, len_lo, len_hi)
    codes, scales = [], []
    for t in (q, k, v):
        sc = float(t.float().abs().max()) / 448.0
        c = torch.empty(t.shape, dtype=torch.uint8)
        flat, src = c.view(-1), t.view(-1)
        for s0 in range(0, src.numel(), 1 << 26):  # bounded host memory
            s1 = min(src.numel(), s0 + (1 << 26))
            flat[s0:s1] = (src[s0:s1].float() / sc).to(torch.float8_e4m3fn).view(torch.uint8)
        codes.append(c)
        scales.append(sc)
    return codes[0], codes[1], codes[2], tuple(scales), seq_lens


def output_gradient(B, H, N, d, dtype="bf16", seed=0):
    """dO [B, H, N, d] on the CPU, from its own generator (seed + 1000)."""
    return _randn((B, H, N, d), _gen(int(seed) + 1000), _DTYPES[dtype])


def varlen_lengths(B, lo, hi, gen):
    """B int32 lengths uniform in [lo, hi]."""
    return torch.randint(int(lo), int(hi) + 1, (B,), generator=gen, dtype=torch.int64).to(torch.int32)


def _block_table(nblk, gen, spare_blocks=0, pool_blocks=None):
    """(block_table [S, max_blocks] int32, pool size): distinct ids placed by a random permutation
    of sum(nblk) + spare_blocks blocks, or, with ``pool_blocks``, ids drawn uniformly with
    replacement from [0, pool_blocks).  Unused entries are -1."""
    S = len(nblk)
    max_blocks = max(1, max(nblk))
    used = sum(nblk)
    if pool_blocks is None:
        pool = used + int(spare_blocks)
        ids = torch.randperm(max(pool, 1), generator=gen, dtype=torch.int64)[:pool]
    else:
        pool = int(pool_blocks)
        if pool <= 0:
            raise ValueError("pool_blocks must be positive")
        ids = torch.randint(0, pool, (used,), generator=gen, dtype=torch.int64)
    table = torch.full((S, max_blocks), -1, dtype=torch.int32)
    pos = 0
    for b, n in enumerate(nblk):
        table[b, :n] = ids[pos:pos + n].to(torch.int32)
        pos += n
    return table, pool


def paged_decode_inputs(S, Hq, Hkv, d, block_size=16, len_lo=512, len_hi=32768, seed=0,
                        seq_lens=None, spare_blocks=0, pool_blocks=None):
    """(q, k_cache, v_cache, block_table, seq_lens) on the CPU, bf16 data, int32 indices.

    ``seq_lens`` may be given explicitly (a list); otherwise it is drawn.  ``spare_blocks``
    adds unreferenced blocks to the pool (their ids are shuffled in with the used ones).
    ``pool_blocks`` switches to a shared pool of that many blocks with ids drawn with
    replacement (``spare_blocks`` is then ignored).
    """
    g = _gen(seed)
    if seq_lens is None:
        lens = torch.randint(int(len_lo), int(len_hi) + 1, (S,), generator=g, dtype=torch.int64)
    else:
        lens = torch.as_tensor(list(seq_lens), dtype=torch.int64)
        if lens.numel() != S:
            raise ValueError("seq_lens must have S entries")
    nblk = [int(math.ceil(int(x) / block_size)) for x in lens]
    table, pool = _block_table(nblk, g, spare_blocks, pool_blocks)
    q = _randn((S, Hq, d), g, torch.bfloat16)
    k_cache = _randn((max(pool, 1), block_size, Hkv, d), g, torch.bfloat16)
    v_cache = _randn((max(pool, 1), block_size, Hkv, d), g, torch.bfloat16)
    return q, k_cache, v_cache, table, lens.to(torch.int32)


def paged_prefill_inputs(S, Hq, Hkv, d, max_q, block_size=16, len_lo=512, len_hi=32768, seed=0,
                         seq_lens=None, q_lens=None, spare_blocks=0, pool_blocks=None):
    """(q [S,Hq,max_q,d], k_cache, v_cache, block_table, seq_lens, q_lens) on the CPU.
    ``pool_blocks`` as for ``paged_decode_inputs``."""
    g = _gen(seed)
    if seq_lens is None:
        lens = torch.randint(int(len_lo), int(len_hi) + 1, (S,), generator=g, dtype=torch.int64)
    else:
        lens = torch.as_tensor(list(seq_lens), dtype=torch.int64)
    nblk = [int(math.ceil(int(x) / block_size)) for x in lens]
    table, pool = _block_table(nblk, g, spare_blocks, pool_blocks)
    q = _randn((S, Hq, max_q, d), g, torch.bfloat16)
    k_cache = _randn((max(pool, 1), block_size, Hkv, d), g, torch.bfloat16)
    v_cache = _randn((max(pool, 1), block_size, Hkv, d), g, torch.bfloat16)
    if q_lens is None:
        ql = [int(torch.randint(1, max(1, min(max_q, int(L))) + 1, (1,), generator=g)) if int(L) > 0
              else 0 for L in lens]
    else:
        ql = list(q_lens)
    return q, k_cache, v_cache, table, lens.to(torch.int32), torch.as_tensor(ql, dtype=torch.int32)
