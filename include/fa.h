/*
 * fa.h -- C ABI of the MI355X (gfx950) fused attention library (libfa.so).
 *
 * Six operations, all asynchronous on the caller's HIP stream:
 *
 *   fa_fwd           fused, tiled attention forward O = softmax(scale * Q K^T) V with an
 *                    online softmax; the N x N score and probability matrices never reach
 *                    device memory.  Also writes the per-row log-sum-exp.
 *   fa_fwd_fp8       the same forward with FP8 (e4m3) q, k, v and per-tensor scales, both
 *                    products on the FP8 matrix cores.
 *   fa_bwd           the matching backward (dQ, dK, dV), recomputing the probabilities from
 *                    the stored log-sum-exp.
 *   fa_paged_decode  one query token per sequence against a KV cache stored in fixed-size
 *                    physical blocks that a block table addresses (non-contiguous gather).
 *   fa_paged_prefill a chunk of each sequence's newest tokens against the same paged cache.
 *   fa_fwd_unfused   the standard three-kernel forward (S and P through device memory), the
 *                    baseline the fused kernel is measured against.
 *
 * Conventions for every entry point
 *   - Every data pointer is a caller-owned DEVICE pointer (e.g. from torch).  The library
 *     allocates nothing, never synchronises the host and never prints.  It keeps no state
 *     between calls, except the static device scratch behind fa_paged_decode_noalloc (held per
 *     GPU for the life of the process).  It is safe to capture in a HIP graph.
 *   - Results are valid once the caller has synchronised `stream` (a hipStream_t; NULL means
 *     the default stream).
 *   - Errors are reported through the return value only.  Argument validation happens before
 *     any HIP call, so an invalid call has no side effect on the device.
 *   - Values that live in device memory (sequence lengths, block ids) cannot be checked
 *     without a synchronisation, so the kernels make them safe instead: sequence lengths are
 *     clamped to their valid range, and a block id outside [0, num_blocks) is never
 *     dereferenced -- that block's keys and values read as zeros.
 *   - All tensors are dense, row-major, with no padding between rows.  Data pointers must be
 *     16-byte aligned.
 *   - Sequence lengths (N, max_q, max_blocks_per_seq * block_size) above 2^30 - 1, and sizes
 *     whose grid of workgroups would not fit a 32-bit count, return FA_ERR_UNSUPPORTED.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null required pointer, non-positive size, H % Hkv != 0,
                             misaligned pointer, negative or non-finite scale,
                             workspace too small, ... */
  FA_ERR_UNSUPPORTED = 2, /* valid but not implemented: head dim not 64/128, unknown dtype,
                             block size not 16, query-group size above 16, ... */
  FA_ERR_HIP = 3,         /* the HIP runtime reported an error (no device, launch failure) */
  FA_ERR_TOO_LARGE = 4    /* fa_paged_decode_noalloc: the sizes need more than the library's
                             static scratch (FA_DECODE_SCRATCH_BYTES) */
} fa_status;

/* Element type of q, k, v and o for fa_fwd. */
enum { FA_BF16 = 0, /* bf16 storage, fp32 arithmetic and accumulation on the matrix cores */
       FA_F32 = 1   /* fp32 storage and fp32 arithmetic throughout */ };

/*
 * fa_fwd -- attention forward.
 *
 * Computes, for every batch b and query head h (kv head g = h / (H / Hkv)):
 *   S = scale * Q[b,h] K[b,g]^T,  P = softmax over each row of S,  O[b,h] = P V[b,g]
 * as defined on the "GPU优化" tag page (guijiagi.com), excerpt "Flash Attention解决了什么问题？",
 * algorithm part, with the scale passed explicitly (1/sqrt(d) for the standard layer).  The
 * kernel follows the fused, tiled scheme of "Gemini 3 Flash的注意力内核重写：算子融合如何实现
 * 亚毫秒级推理" (sections on kernel fusion, tiling and the online softmax) and the running
 * statistics of "FlashAttention优化" §3.2.1: a row maximum m and row sum l, the output
 * normalised once at the end.  (Each row's reference m is taken from its first key tile and kept;
 * a workgroup in which some later probability could exceed 2^16 recomputes with the running
 * maximum and rescaling of §3.2.1.  Both give the same softmax.)
 *
 *   q         [B, H, N, d]    element type `dtype`
 *   k, v      [B, Hkv, N, d]  element type `dtype`
 *   o         [B, H, N, d]    element type `dtype`, written
 *   lse       [B, H, N] fp32, written: natural-log log-sum-exp of the scaled scores of each
 *             row, max_j(S_ij) + ln(sum_j exp(S_ij - max_j S_ij)) -- the per-row statistic a
 *             recompute backward needs (page "Gemini 3 Flash的注意力内核重写", §4 on
 *             recomputation keeps each row's maximum and normaliser).
 *   B, H, Hkv, N  > 0, H % Hkv == 0 (grouped-query heads share kv heads in consecutive groups;
 *             "FlashAttention优化" §5.3).
 *   d         head dimension: 64 or 128.
 *   scale     finite and >= 0.
 *   causal    nonzero: key j is visible to query i only if j <= i (square, diagonal kept).
 *   seq_lens  NULL, or a device int32[B] of valid lengths L_b (clamped to [0, N]): keys
 *             j >= L_b are masked and query rows i >= L_b are padding, written as O = 0 and
 *             lse = -inf.  Combines with `causal`.
 *   dtype     FA_BF16 or FA_F32.
 *   stream    hipStream_t or NULL.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int Hkv, int N, int d, float scale, int causal, const int32_t* seq_lens,
                 int dtype, void* stream);

/*
 * fa_fwd_fp8 -- attention forward from FP8 inputs.
 *
 * The FP8 variant of fa_fwd (FP8 tensor-core attention is what the "GPU优化" tag page,
 * excerpt "注意力计算的性能瓶颈", credits FlashAttention V3 with).  q, k, v hold e4m3 codes
 * (OCP e4m3fn: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, largest
 * finite value 448); the tensor they stand for is the descale factor times the decoded codes,
 * Q = q_scale * e4m3(q) and likewise K, V.  Computes O = softmax(scale * Q K^T) V and the LSE
 * as fa_fwd does, with these differences in arithmetic:
 *   - both products run on the FP8 matrix cores with fp32 accumulation;
 *   - the softmax runs over blocks of 64 keys with the online recurrence of
 *     "FlashAttention优化" §3.2.1, where each row's reference m moves to a block's maximum only
 *     when that maximum exceeds it by more than a factor 2^2 (so exp(S - m) <= 4); the
 *     probabilities of a block enter the P V product as e4m3(64 p) / 64 (relative error at most
 *     2^-4 each), while the row sum and the LSE use them unrounded.
 *
 *   q         [B, H, N, d] e4m3 codes (1 byte each)
 *   k, v      [B, Hkv, N, d] e4m3 codes
 *   q_scale, k_scale, v_scale  descale factors, finite and >= 0
 *   o         [B, H, N, d] bf16, written (0 for padding rows)
 *   lse       [B, H, N] fp32, written, as for fa_fwd (-inf for padding rows)
 *   B, H, Hkv, N, d, scale, causal, seq_lens, stream: as for fa_fwd (d: 64 or 128).
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale,
                     float v_scale, void* o, float* lse, int B, int H, int Hkv, int N, int d,
                     float scale, int causal, const int32_t* seq_lens, void* stream);

/*
 * fa_bwd_workspace_bytes -- size in bytes of the device workspace fa_bwd needs: two fp32
 * per query row, D = rowsum(dO * O) and the LSE in base 2, each array rounded up to 256 bytes.
 * Returns 0 for non-positive sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/*
 * fa_bwd -- attention backward by recomputation.
 *
 * Gradients of O = softmax(scale * Q K^T) V (as defined for fa_fwd) with respect to Q, K and
 * V, given the output gradient dO.  The probabilities are not stored by the forward: they are
 * recomputed from q, k and the forward's per-row lse, P = exp(scale * Q K^T - lse) (page
 * "Gemini 3 Flash的注意力内核重写", §4 on recomputation: the forward keeps each row's maximum
 * and normaliser so that the backward can rebuild the scores).  With D_i = sum_d dO_id O_id,
 *   dV = P^T dO,   dS = P o (dO V^T - D),   dQ = scale * dS K,   dK = scale * dS^T Q,
 * summed over the query heads of each kv head for dK and dV.
 *
 *   q, o, dout   [B, H, N, d] bf16: the forward's inputs, its output and the output gradient
 *   k, v         [B, Hkv, N, d] bf16
 *   lse          [B, H, N] fp32: the lse fa_fwd wrote for these q, k, v (natural log)
 *   dq           [B, H, N, d] bf16, written (0 for padding rows)
 *   dk, dv       [B, Hkv, N, d] bf16, written (0 for keys at or past the valid length)
 *   B, H, Hkv, N, d, scale, causal, seq_lens: as for fa_fwd (d: 64 or 128).
 *   dtype        FA_BF16 (FA_F32 is not supported by the backward).
 *   workspace    device buffer of at least fa_bwd_workspace_bytes(B, H, N) bytes, 16-byte
 *                aligned, owned by the caller; its contents on entry do not matter.  Calls
 *                that share a workspace must be ordered.
 *   stream       hipStream_t or NULL.
 * The result is deterministic: no atomics, a fixed summation order.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N,
                 int d, float scale, int causal, const int32_t* seq_lens, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_paged_decode_workspace_bytes -- size in bytes of the device workspace fa_paged_decode
 * needs for these sizes (partial outputs and statistics of the key-range splits).  Returns 0
 * for non-positive sizes.
 */
size_t fa_paged_decode_workspace_bytes(int num_seqs, int Hq, int d, int max_blocks_per_seq,
                                       int block_size);

/*
 * fa_paged_decode -- decode attention over a paged KV cache.
 *
 * One query token per sequence attends to all L_b cached tokens of its sequence.  The cache
 * is stored in physical blocks of `block_size` tokens scattered through a pool; token t of
 * sequence b lives in block block_table[b][t / block_size] at slot t % block_size.  The kernel
 * prefetches the block ids into registers, gathers each block's keys and values with
 * coalesced loads through on-chip memory and attends to them in the same kernel, following
 * the non-contiguous block gather page (ocdem.com, vLLM PagedAttention rework) §二.1 (two-stage
 * gather through shared memory), §二.3 (index prefetch into registers) and §二.4 (gather and
 * attention fused).  Long sequences are cut into key ranges processed in parallel whose
 * partial (max, sum, output) triples are merged exactly, as the online-softmax recurrence of
 * "FlashAttention优化" §3.2 allows for any block order.
 *
 *   q            [num_seqs, Hq, d] bf16
 *   k_cache      [num_blocks, block_size, Hkv, d] bf16
 *   v_cache      [num_blocks, block_size, Hkv, d] bf16
 *   block_table  [num_seqs, max_blocks_per_seq] int32 physical block ids in [0, num_blocks);
 *                entries at index >= ceil(L_b / block_size) are never read.  Ids may repeat
 *                (sequences sharing blocks of one pool).  An id outside [0, num_blocks) is not
 *                an error the call can report: its block reads as zeros (keys and values 0).
 *   seq_lens     [num_seqs] int32 (device), clamped to [0, max_blocks_per_seq * block_size].
 *                A sequence of length 0 gives O = 0 and lse = -inf.
 *   o            [num_seqs, Hq, d] bf16, written.
 *   lse          [num_seqs, Hq] fp32, written (natural log, as for fa_fwd), or NULL.
 *   Hq % Hkv == 0 and Hq / Hkv <= 16.  d: 64 or 128.  block_size: 16.
 *   scale        finite and >= 0.
 *   workspace    device buffer of at least fa_paged_decode_workspace_bytes(...) bytes,
 *                16-byte aligned, owned by the caller; its contents on entry do not matter.
 *   stream       hipStream_t or NULL.  Calls that share a workspace must be ordered.
 */
fa_status fa_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens, void* o,
                          float* lse, int num_seqs, int Hq, int Hkv, int d, int block_size,
                          int max_blocks_per_seq, int num_blocks, float scale, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch behind fa_paged_decode_noalloc (per GPU). */
#define FA_DECODE_SCRATCH_BYTES ((size_t)80 << 20)

/*
 * fa_paged_decode_noalloc -- fa_paged_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation.  It
 * takes no workspace: the key-range partials go to a static device array of
 * FA_DECODE_SCRATCH_BYTES that the library holds on every GPU it runs on until the process
 * ends (its address is looked up once per device, on the first call there).  The call
 * allocates nothing and runs the same kernels as fa_paged_decode, so the results are identical.
 *
 *   Arguments: as for fa_paged_decode, without workspace and workspace_bytes.
 *   Sizes: fa_paged_decode_workspace_bytes(num_seqs, Hq, d, max_blocks_per_seq, block_size) must
 *          not exceed FA_DECODE_SCRATCH_BYTES (80 MiB: e.g. 64 sequences x 32 query heads with
 *          a 32768-token block table at d = 128), else FA_ERR_TOO_LARGE before any HIP call.
 *   stream: must belong to the current device (else FA_ERR_HIP).
 *   Calls on one GPU share the scratch: calls that overlap on it (different streams, or
 *   different host threads without ordering) race and must not be issued.  Nothing in the
 *   scratch needs to start at zero; it keeps the last call's partials.
 */
fa_status fa_paged_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens, void* o,
                                  float* lse, int num_seqs, int Hq, int Hkv, int d,
                                  int block_size, int max_blocks_per_seq, int num_blocks,
                                  float scale, void* stream);

/*
 * fa_paged_prefill_workspace_bytes -- size in bytes of the device workspace fa_paged_prefill
 * needs for these sizes: the work plan (a few ints per sequence and per work item) and the
 * partial results of split key ranges, whose number is bounded by a constant (2048 slots of 128
 * query rows, or 1024 of 256 when max_q >= 256, x (d + 2) floats: 130 MiB at d = 128, 66 MiB at
 * d = 64) whatever the lengths.
 * Returns 0 for non-positive sizes or Hq not a multiple of Hkv.
 */
size_t fa_paged_prefill_workspace_bytes(int num_seqs, int max_q, int Hq, int Hkv, int d,
                                        int max_blocks_per_seq);

/*
 * fa_paged_prefill -- chunked prefill against a paged KV cache.
 *
 * For each sequence b the query chunk is its newest Q_b = q_lens[b] tokens, at positions
 * L_b - Q_b .. L_b - 1 of the sequence (L_b = seq_lens[b]), whose keys and values are already
 * in the cache.  Query row i attends to the cached tokens 0 .. L_b - Q_b + i (causal with that
 * offset) -- the chunked prefill of the LLM inference-optimisation article (ijyty.com) §3.2, a
 * long prompt processed piece by piece against the cache built so far; Q_b = 1 is one decode
 * step.  The cache and block table are as for fa_paged_decode; the arithmetic is fa_fwd's, with
 * the key/value tiles gathered block by block through the table.  A small planning kernel reads
 * the lengths on the device and lays out the work; key ranges much longer than the average
 * work per compute unit are split and their partial results merged exactly (the block merge of
 * the online softmax, "FlashAttention优化" §3.2.2), so the result does not depend on the split
 * beyond floating-point rounding.
 *
 *   q            [num_seqs, Hq, max_q, d] bf16 (head-major, as fa_fwd's q); rows i >= Q_b are
 *                padding
 *   k_cache, v_cache, block_table: as for fa_paged_decode
 *   seq_lens     [num_seqs] int32 (device): tokens in the cache, clamped to
 *                [0, max_blocks_per_seq * block_size]
 *   q_lens       [num_seqs] int32 (device): chunk lengths, clamped to [0, min(L_b, max_q)]
 *   o            [num_seqs, Hq, max_q, d] bf16, written (0 in padding rows)
 *   lse          [num_seqs, Hq, max_q] fp32, written (natural log; -inf in padding rows)
 *   Hq % Hkv == 0.  d: 64 or 128.  block_size: 16.  scale finite and >= 0.
 *   workspace    device buffer of at least fa_paged_prefill_workspace_bytes(num_seqs, max_q,
 *                Hq, Hkv, d, max_blocks_per_seq) bytes, 16-byte aligned, owned by the caller;
 *                its contents on entry do not matter (smaller: FA_ERR_INVALID_ARG).
 *   stream       hipStream_t or NULL.  Calls that share a workspace must be ordered.
 */
fa_status fa_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* q_lens, void* o, float* lse, int num_seqs, int max_q,
                           int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq,
                           int num_blocks, float scale, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * fa_fwd_unfused_workspace_bytes -- bytes of the workspace fa_fwd_unfused needs: the N x N
 * score matrix in fp32 and the probability matrix in bf16 for every (batch, head).
 */
size_t fa_fwd_unfused_workspace_bytes(int B, int H, int N);

/*
 * fa_fwd_unfused -- the standard, unfused attention forward, kept as the baseline the fused
 * kernel is measured against ("FlashAttention优化" §2.1-§2.2: S = scale * Q K^T written to
 * device memory, a three-pass softmax reading S and writing P, then O = P V reading P).  Same
 * result as fa_fwd (bf16, no padding lengths) at the cost of the N x N round trips.
 *
 *   q, k, v, o, lse, B, H, Hkv, d, scale, causal: as for fa_fwd (bf16 only).
 *   N            a multiple of 8.
 *   workspace    device buffer of at least fa_fwd_unfused_workspace_bytes(B, H, N) bytes,
 *                16-byte aligned, owned by the caller (6 * B * H * N^2 bytes).
 *   stream       hipStream_t or NULL.
 */
fa_status fa_fwd_unfused(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H, int Hkv, int N, int d, float scale, int causal, void* workspace,
                         size_t workspace_bytes, void* stream);

/* fa_status_str -- static, NUL-terminated description of a status code. */
const char* fa_status_str(fa_status status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
