"""Flop and byte accounting for the attention kernels (host-side arithmetic only).

The counts are the algorithmic ones the throughput figures are quoted in:
* forward flops: two contractions of 2*N*N*d each per (batch, head), i.e. 4*B*H*N^2*d,
  halved under causal masking; with per-sequence lengths the sum over sequences of
  4*H*L_b^2*d (halved under causal).
* chunked prefill flops: 4*Hq*d per visible (query, key) pair; the chunk of Q_b rows at offset
  L_b - Q_b sees Q_b*(L_b - Q_b) + Q_b*(Q_b + 1)/2 pairs.
* backward flops: five contractions of the same size (S = Q K^T recomputed, dV = P^T dO,
  dP = dO V^T, dQ = dS K, dK = dS^T Q), i.e. 2.5 times the forward's.
* decode bytes: every cached K and V element a step must read (sum of L_b*Hkv*d*2 bytes for
  each of K and V), plus q, o, lse, the block ids in use and the lengths.

``score_matrix_bytes`` and ``qkv_bytes`` reproduce the sizes the pages print for the
intermediate N x N matrix of unfused attention ("Gemini 3 Flash的注意力内核重写", section on
the memory-bandwidth bottleneck of standard attention; "FlashAttention优化" §2.1; the
"GPU优化" tag page's excerpts on the 128K attention matrix and the n=8192 score matrix).
"""

import math

__all__ = [
    "attention_flops",
    "attention_bwd_flops",
    "paged_prefill_flops",
    "forward_min_bytes",
    "decode_bytes",
    "decode_flops",
    "score_matrix_bytes",
    "qkv_bytes",
    "kv_cache_bytes",
    "MI355X_BF16_DENSE_TFLOPS",
    "MI355X_FP8_DENSE_TFLOPS",
    "MI355X_HBM_GBPS",
    "MI355X_PEAK_MHZ",
]

MI355X_BF16_DENSE_TFLOPS = 2500.0   # published dense bf16 matrix peak
MI355X_FP8_DENSE_TFLOPS = 5000.0    # published dense fp8 matrix peak
MI355X_HBM_GBPS = 8000.0            # published HBM3E peak
MI355X_PEAK_MHZ = 2400.0            # engine clock the published matrix peaks assume


def attention_flops(B, H, N, d, causal=False, seq_lens=None):
    """Algorithmic flops of one forward pass (QK^T and PV contractions only)."""
    if seq_lens is None:
        f = 4 * B * H * N * N * d
    else:
        f = sum(4 * H * int(L) * int(L) * d for L in seq_lens)
    return f / 2 if causal else f


def attention_bwd_flops(B, H, N, d, causal=False, seq_lens=None):
    """Algorithmic flops of one backward pass: five contractions, 2.5x the forward's."""
    return 2.5 * attention_flops(B, H, N, d, causal=causal, seq_lens=seq_lens)


def paged_prefill_flops(seq_lens, q_lens, Hq, d):
    """Algorithmic flops of one chunked prefill against the paged cache."""
    pairs = sum(int(Q) * (int(L) - int(Q)) + int(Q) * (int(Q) + 1) // 2
                for L, Q in zip(seq_lens, q_lens))
    return 4 * Hq * d * pairs


def forward_min_bytes(B, H, Hkv, N, d, elem_bytes=2):
    """Compulsory HBM bytes of one fused forward: read q, k, v once, write o and fp32 lse."""
    return (B * H * N * d * 2 + 2 * B * Hkv * N * d) * elem_bytes + B * H * N * 4


def decode_bytes(seq_lens, Hq, Hkv, d, block_size=16, elem_bytes=2):
    """Algorithmic bytes of one paged decode step."""
    S = len(seq_lens)
    kv = sum(int(L) for L in seq_lens) * Hkv * d * elem_bytes * 2
    qo = 2 * S * Hq * d * elem_bytes
    lse = S * Hq * 4
    ids = sum(int(math.ceil(int(L) / block_size)) for L in seq_lens) * 4
    return kv + qo + lse + ids + S * 4


def decode_flops(seq_lens, Hq, d):
    return sum(4 * int(L) * Hq * d for L in seq_lens)


def score_matrix_bytes(N, heads=1, elem_bytes=2):
    """Bytes of the materialised N x N score matrix (the unfused path's intermediate)."""
    return N * N * heads * elem_bytes


def qkv_bytes(N, d, elem_bytes=2):
    """Bytes of Q, K and V for one head."""
    return 3 * N * d * elem_bytes


def kv_cache_bytes(layers, heads, head_dim, seq_len, batch, elem_bytes=2):
    """KV-cache size: one K and one V element per (layer, head, dim, token, sequence)."""
    return 2 * layers * heads * head_dim * seq_len * batch * elem_bytes
