// fa_launch.h -- internal interface between the C-ABI layer (fa_api.cpp) and the kernels.
// Arguments are already validated when these run; each returns the HIP launch status.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "fa.h"
#include "fa_prefill_plan.h"

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* seq_lens;  // nullptr: every sequence has N valid rows
  int B, H, Hkv, N, d;
  float scale;
  bool causal;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);

struct Fp8FwdArgs {
  const void* q;  // e4m3 codes
  const void* k;
  const void* v;
  float q_scale, k_scale, v_scale;  // per-tensor descale factors
  void* o;                          // bf16
  float* lse;
  const int32_t* seq_lens;
  int B, H, Hkv, N, d;
  float scale;
  bool causal;
};

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;  // may be nullptr
  int S, Hq, Hkv, d, block_size, max_blocks, num_blocks;
  float scale;
  void* workspace;
};

struct UnfusedArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  void* workspace;  // S fp32 [B, H, N, N], then P bf16 [B, H, N, N]
  int B, H, Hkv, N, d;
  float scale;
  bool causal;
};

size_t unfused_workspace_bytes(int B, int H, int N);
hipError_t launch_fwd_unfused(const UnfusedArgs& a, hipStream_t stream);

struct PagedPrefillArgs {
  const void* q;  // [S, Hq, max_q, d]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* q_lens;
  void* o;     // [S, Hq, max_q, d]
  float* lse;  // [S, Hq, max_q]
  int S, max_q, Hq, Hkv, d, max_blocks, num_blocks;
  float scale;
  void* workspace;  // paged_prefill_workspace_bytes(...) bytes: the plan and the split partials
};

// The work plan's shape for these sizes (heads per work item, rows per head, resident
// workgroups) and the workspace it needs; 0 for non-positive sizes.
plan::Shape paged_prefill_shape(int S, int max_q, int Hq, int Hkv, int max_blocks);
size_t paged_prefill_workspace_bytes(int S, int max_q, int Hq, int Hkv, int d, int max_blocks);
hipError_t launch_paged_prefill(const PagedPrefillArgs& a, hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  const int32_t* seq_lens;  // nullptr: every sequence has N valid rows
  void* workspace;          // D = rowsum(dO * O) [B, H, N] fp32
  int B, H, Hkv, N, d;
  float scale;
  bool causal;
};

size_t bwd_workspace_bytes(int B, int H, int N);
// Floats in one per-row statistics array (D or the base-2 LSE) of the backward's workspace.
size_t bwd_stat_floats(int B, int H, int N);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);

// Tokens per key-range split of the decode kernel (512, or 1024 when the block table holds at
// least kLongSplitMinRanges such ranges and the grid of 1024-token ranges has at least
// kLongSplitMinWaves waves: four rounds of the 1280 waves the chip holds at once, five 32 KB
// rings per CU), key ranges per sequence in its grid, and the resulting workspace size.
// decode_splits counts 512-token ranges, the larger count, so the workspace and the grid-size
// check hold for either length.
constexpr int kDecodeSplitTokens = 512;
constexpr int kDecodeLongSplitTokens = 1024;
constexpr int kLongSplitMinRanges = 8;
constexpr long long kLongSplitMinWaves = 4LL * 5 * 256;
int decode_splits(int max_blocks, int block_size);
int decode_splits_of(int max_blocks, int block_size, int split);
size_t decode_workspace_bytes(int S, int Hq, int d, int max_blocks, int block_size);
hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream);

// The decode with its partials in the library's static device scratch (a.workspace is ignored):
// kDecodeScratchBytes per GPU, so decode_workspace_bytes(...) must not exceed it.
constexpr size_t kDecodeScratchBytes = FA_DECODE_SCRATCH_BYTES;
hipError_t launch_paged_decode_noalloc(DecodeArgs a, hipStream_t stream);

}  // namespace fa
