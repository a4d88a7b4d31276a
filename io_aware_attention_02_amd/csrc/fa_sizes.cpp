// fa_sizes.cpp -- host-side size arithmetic of the library: workspace sizes and the decode's
// key-range count.  Plain C++ with no device code, shared by the C-ABI layer (fa_api.cpp) and
// the launchers, so that the argument validation builds and runs without the GPU toolchain.
#include <cstddef>
#include <cstdint>

#include "fa_launch.h"

namespace fa {
namespace {
constexpr int kXcdsHost = 8;  // accelerator complex dies of an MI355X
constexpr int kCUsHost = 256;   // compute units of an MI355X
constexpr int kWaveRows = 32;   // query rows per wave of the forward kernels
// The chunked prefill's attention workgroups have eight waves (one per CU, sharing each key and
// value tile, as the contiguous forward's 256-row workgroups do) when the chunk tensor holds at
// least this many rows per head, else four (two per CU): items of 64 rows per head would leave
// most waves idle on short chunks.
constexpr int kPrefillWideRows = 256;

// Query heads per work item of the chunked prefill: the largest of 4, 2, 1 dividing the group.
int heads_per_item(int group) { return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1); }
}  // namespace

// Floats in one per-row statistics array (D or the base-2 LSE) of the backward's workspace,
// rounded up to 256 bytes.
size_t bwd_stat_floats(int B, int H, int N) { return ((size_t)B * H * N + 63) / 64 * 64; }

size_t bwd_workspace_bytes(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return 2 * bwd_stat_floats(B, H, N) * sizeof(float);
}

// The unfused forward's workspace: S in fp32 and P in bf16 for every (batch, head).
size_t unfused_workspace_bytes(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return (size_t)B * H * N * N * (sizeof(float) + sizeof(uint16_t));
}

// Key ranges per sequence in the split grid (the workspace holds one partial result per range):
// ceil(max tokens / range length), raised to 7 mod 8 once there are at least 8.  Work unit u = b * MS + sp
// runs on XCD u mod 8 (workgroups are dealt round-robin over the XCDs), so with MS = 7 mod 8,
// range sp of sequence b lands on XCD (sp - b) mod 8: each sequence starts on a different XCD,
// and the ranges left over after whole rounds of 8 (and the empty ones past a short sequence's
// end) spread over all XCDs instead of piling onto the low-numbered ones.  The added ranges are
// empty and exit at once.
int decode_splits_of(int max_blocks, int block_size, int split) {
  const long long tokens = (long long)max_blocks * block_size;
  int ms = (int)((tokens + split - 1) / split);
  if (ms >= kXcdsHost) ms += kXcdsHost - 1 - ms % kXcdsHost;
  return ms;
}

// The 512-token count bounds the 1024-token one (both steps are monotone in the token count), so
// the workspace and the grid-size check use it whichever length the launch picks.
int decode_splits(int max_blocks, int block_size) {
  return decode_splits_of(max_blocks, block_size, kDecodeSplitTokens);
}

size_t decode_workspace_bytes(int S, int Hq, int d, int max_blocks, int block_size) {
  if (S <= 0 || Hq <= 0 || d <= 0 || max_blocks <= 0 || block_size <= 0) return 0;
  const size_t slots = (size_t)S * Hq * decode_splits(max_blocks, block_size);
  return slots * ((size_t)d + 2) * sizeof(float);
}

plan::Shape paged_prefill_shape(int S, int max_q, int Hq, int Hkv, int max_blocks) {
  const int hp = heads_per_item(Hq / Hkv);
  plan::Shape s;
  s.S = S;
  s.max_q = max_q;
  s.Hkv = Hkv;
  s.hgk = Hq / Hkv / hp;
  const int nw = max_q >= kPrefillWideRows ? 8 : 4;  // waves per attention workgroup
  s.pairs = kWaveRows * nw;
  s.rph = s.pairs / hp;
  s.max_keys = max_blocks * plan::kPageRows;
  s.R = kCUsHost * 8 / nw;  // resident workgroups: one or two per CU
  return s;
}

size_t paged_prefill_workspace_bytes(int S, int max_q, int Hq, int Hkv, int d, int max_blocks) {
  if (S <= 0 || max_q <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_blocks <= 0 || Hq % Hkv != 0)
    return 0;
  return plan::layout(paged_prefill_shape(S, max_q, Hq, Hkv, max_blocks), d).total;
}

}  // namespace fa
