// fa_api.cpp -- the C ABI of libfa.so (declared in include/fa.h).
//
// Every entry point validates its arguments completely before touching the HIP runtime, so
// a rejected call has no device-side effect, then launches the kernels on the caller's
// stream and reports the launch status.  Nothing here allocates, synchronises or prints.
#include "fa.h"

#include <hip/hip_runtime_api.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "fa_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_scale(float s) { return std::isfinite(s) && s >= 0.f; }

// Sequence positions (and position + tile size) stay in 32-bit integers inside the kernels.
constexpr int kMaxN = INT_MAX / 2;

// a * b * c <= limit for positive factors, decided without overflowing.
bool product_at_most(long long limit, long long a, long long b, long long c) {
  return a <= limit / b && a * b <= limit / c;
}

}  // namespace

extern "C" {

const char* fa_status_str(fa_status status) {
  switch (status) {
    case FA_OK:
      return "ok";
    case FA_ERR_INVALID_ARG:
      return "invalid argument";
    case FA_ERR_UNSUPPORTED:
      return "unsupported configuration";
    case FA_ERR_HIP:
      return "HIP runtime error";
    case FA_ERR_TOO_LARGE:
      return "sizes exceed the static scratch of the no-allocation entry point";
  }
  return "unknown status";
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int Hkv, int N, int d, float scale, int causal, const int32_t* seq_lens,
                 int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return FA_ERR_INVALID_ARG;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // One workgroup per (batch, head, query tile of >= 32 rows) must fit a 1-D grid.
  if (N > kMaxN || !product_at_most(INT_MAX, B, H, (N + 31) / 32)) return FA_ERR_UNSUPPORTED;

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.seq_lens = seq_lens;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == FA_BF16 ? fa::launch_fwd_bf16(a, s) : fa::launch_fwd_f32(a, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale,
                     float v_scale, void* o, float* lse, int B, int H, int Hkv, int N, int d,
                     float scale, int causal, const int32_t* seq_lens, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!valid_scale(scale) || !valid_scale(q_scale) || !valid_scale(k_scale) ||
      !valid_scale(v_scale))
    return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (N > kMaxN || !product_at_most(INT_MAX, B, H, (N + 127) / 128)) return FA_ERR_UNSUPPORTED;
  fa::Fp8FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.o = o;
  a.lse = lse;
  a.seq_lens = seq_lens;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  const hipError_t e = fa::launch_fwd_fp8(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fwd_unfused_workspace_bytes(int B, int H, int N) {
  return fa::unfused_workspace_bytes(B, H, N);
}

fa_status fa_fwd_unfused(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H, int Hkv, int N, int d, float scale, int causal, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (N % 8 != 0) return FA_ERR_UNSUPPORTED;  // aligned 16-byte score and 8-byte P accesses
  // Grids: one workgroup per (batch, head, 128 rows), and one per 4 rows of the softmax pass.
  if (N > kMaxN || !product_at_most(INT_MAX, B, H, (N + 127) / 128) ||
      !product_at_most(4LL * (INT_MAX - 1), B, H, N))
    return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fa::unfused_workspace_bytes(B, H, N)) return FA_ERR_INVALID_ARG;
  fa::UnfusedArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.workspace = workspace;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  const hipError_t e = fa::launch_fwd_unfused(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_paged_prefill_workspace_bytes(int num_seqs, int max_q, int Hq, int Hkv, int d,
                                        int max_blocks_per_seq) {
  return fa::paged_prefill_workspace_bytes(num_seqs, max_q, Hq, Hkv, d, max_blocks_per_seq);
}

fa_status fa_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* q_lens, void* o, float* lse, int num_seqs, int max_q,
                           int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq,
                           int num_blocks, float scale, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !q_lens || !o || !lse ||
      !workspace)
    return FA_ERR_INVALID_ARG;
  if (num_seqs <= 0 || max_q <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0)
    return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) || (reinterpret_cast<uintptr_t>(q_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) || !aligned16(workspace))
    return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (block_size != 16) return FA_ERR_UNSUPPORTED;
  // Key positions and offsets in 32-bit integers; the work items (sequence x kv head x head
  // subset x query block, at least 32 rows per block) indexed by 32-bit integers, 8 per item.
  if (max_q > kMaxN || (long long)max_blocks_per_seq * block_size > kMaxN ||
      !product_at_most(INT_MAX / 16, num_seqs, Hq, (max_q + 31) / 32))
    return FA_ERR_UNSUPPORTED;
  if (workspace_bytes <
      fa::paged_prefill_workspace_bytes(num_seqs, max_q, Hq, Hkv, d, max_blocks_per_seq))
    return FA_ERR_INVALID_ARG;

  fa::PagedPrefillArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.q_lens = q_lens;
  a.o = o;
  a.lse = lse;
  a.S = num_seqs;
  a.max_q = max_q;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.scale = scale;
  a.workspace = workspace;
  const hipError_t e = fa::launch_paged_prefill(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(int B, int H, int N) { return fa::bwd_workspace_bytes(B, H, N); }

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N,
                 int d, float scale, int causal, const int32_t* seq_lens, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
    return FA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return FA_ERR_INVALID_ARG;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;  // unknown, or fp32 (forward only)
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // Grids: one workgroup per (batch, head, 128 rows), and one per 16 rows of the row pass.
  if (N > kMaxN || !product_at_most(INT_MAX, B, H, (N + 127) / 128) ||
      !product_at_most(16LL * (INT_MAX - 1), B, H, N))
    return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fa::bwd_workspace_bytes(B, H, N)) return FA_ERR_INVALID_ARG;

  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.seq_lens = seq_lens;
  a.workspace = workspace;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  const hipError_t e = fa::launch_bwd_bf16(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_paged_decode_workspace_bytes(int num_seqs, int Hq, int d, int max_blocks_per_seq,
                                       int block_size) {
  return fa::decode_workspace_bytes(num_seqs, Hq, d, max_blocks_per_seq, block_size);
}

}  // extern "C"

namespace {

// Checks shared by both decode entry points (everything except the workspace) and the packed
// launch arguments; returns FA_OK when the call may proceed.
fa_status check_decode(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                       int num_seqs, int Hq, int Hkv, int d, int block_size,
                       int max_blocks_per_seq, int num_blocks, float scale, fa::DecodeArgs* a) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o) return FA_ERR_INVALID_ARG;
  if (num_seqs <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0)
    return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (block_size != 16) return FA_ERR_UNSUPPORTED;
  if (Hq / Hkv > 16) return FA_ERR_UNSUPPORTED;
  // Grid: one 64-thread workgroup per (kv head, key range, sequence), at most one per 512
  // tokens, rounded up to a multiple of 8 ranges; the total thread count must fit a 32-bit grid.
  if ((long long)max_blocks_per_seq * block_size > kMaxN) return FA_ERR_UNSUPPORTED;
  const long long splits = fa::decode_splits(max_blocks_per_seq, block_size);
  const long long units = ((long long)num_seqs * splits + 7) / 8 * 8;
  if (!product_at_most(INT_MAX, units, Hkv, 64)) return FA_ERR_UNSUPPORTED;
  a->q = q;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->block_table = block_table;
  a->seq_lens = seq_lens;
  a->o = o;
  a->lse = lse;
  a->S = num_seqs;
  a->Hq = Hq;
  a->Hkv = Hkv;
  a->d = d;
  a->block_size = block_size;
  a->max_blocks = max_blocks_per_seq;
  a->num_blocks = num_blocks;
  a->scale = scale;
  a->workspace = nullptr;
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens, void* o,
                          float* lse, int num_seqs, int Hq, int Hkv, int d, int block_size,
                          int max_blocks_per_seq, int num_blocks, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
  fa::DecodeArgs a;
  const fa_status st = check_decode(q, k_cache, v_cache, block_table, seq_lens, o, lse, num_seqs,
                                    Hq, Hkv, d, block_size, max_blocks_per_seq, num_blocks, scale,
                                    &a);
  if (st != FA_OK) return st;
  if (!workspace || !aligned16(workspace)) return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa::decode_workspace_bytes(num_seqs, Hq, d, max_blocks_per_seq, block_size))
    return FA_ERR_INVALID_ARG;
  a.workspace = workspace;
  const hipError_t e = fa::launch_paged_decode(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_paged_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens, void* o,
                                  float* lse, int num_seqs, int Hq, int Hkv, int d,
                                  int block_size, int max_blocks_per_seq, int num_blocks,
                                  float scale, void* stream) {
  fa::DecodeArgs a;
  const fa_status st = check_decode(q, k_cache, v_cache, block_table, seq_lens, o, lse, num_seqs,
                                    Hq, Hkv, d, block_size, max_blocks_per_seq, num_blocks, scale,
                                    &a);
  if (st != FA_OK) return st;
  if (fa::decode_workspace_bytes(num_seqs, Hq, d, max_blocks_per_seq, block_size) >
      fa::kDecodeScratchBytes)
    return FA_ERR_TOO_LARGE;
  const hipError_t e = fa::launch_paged_decode_noalloc(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
