// fa_decode.hip -- decode attention over a paged KV cache (one query token per sequence).
//
// The cache is a pool of physical blocks of 16 tokens, [num_blocks][16][Hkv][d]; a block
// table maps each sequence's logical blocks to physical ones.  Following the non-contiguous
// block gather page (ocdem.com, vLLM PagedAttention rework):
//  * §二.3 -- the block ids a wave will visit are loaded into registers up front (one id per
//    lane) and read from there into scalar registers, so no gather waits on the index array;
//  * §二.1 -- each block's values are gathered with coalesced direct loads into on-chip memory
//    (a ring of stages), and read from there in the layout the matrix cores want;
//  * §二.4 -- gather and attention are one kernel: scores against the register-resident query,
//    online softmax and the probability-weighted sum of values follow each gathered block.
// Load balance (§二.2 asks for dynamic balancing of unequal per-query work): instead of a
// per-warp task queue, each sequence's tokens are cut into fixed-length ranges (512 tokens, or
// 1024 when the grid is large enough to fill the chip with them), one wave each, so work per wave
// is equal whatever the length mix.  Each range writes its partial
// (max, sum, unnormalised output); a second kernel merges them exactly with the rescaling
// rule of the online softmax ("FlashAttention优化" §3.2.2: the result is the same for any
// block order and grouping).
//
// CDNA4 mapping:
//  * The Hq/Hkv query heads sharing kv head g are the 16 columns of the matrix-core tiles
//    (unused columns are zero).  Scores S^T = K Q^T with v_mfma_f32_16x16x32_bf16; P^T is the
//    score accumulator packed to bf16, the B operand of O^T += V^T P^T
//    (v_mfma_f32_16x16x16_bf16), so probabilities never leave registers.
//  * K and V go from global memory straight into LDS (buffer_load ... lds, 16 bytes per lane):
//    each load instruction covers whole token rows, so it requests whole cache lines.  Chunks are
//    XOR-swizzled by row so that the fragment reads are free of bank conflicts: K fragments
//    (one token row, 8 head dims per lane and MFMA step) with ds_read_b128, V^T fragments with
//    ds_read_b64_tr_b16.
//  * Every load is issued kStages-1 blocks ahead of its use through a per-block buffer
//    resource whose size ends at the sequence length: cache slots past the length read as
//    zeros (never as whatever the pool holds there) and no load leaves the block.
#include "fa_device.h"
#include "fa_launch.h"

#include <mutex>

namespace fa {
namespace {

typedef __attribute__((address_space(3))) char lds_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBS = 16;                         // tokens per physical block
constexpr int kSplit = kDecodeSplitTokens;      // tokens per wave, short grids
constexpr int kLongSplit = kDecodeLongSplitTokens;  // tokens per wave, long grids
constexpr int kBlocksPerSplit = kLongSplit / kBS;  // block ids prefetched per wave (<= 64)
constexpr int kStages = 4;                      // blocks in the load ring
constexpr int kBufferFlags = 0x00020000;        // buffer resource word 3: 32-bit data, raw
constexpr int kXcds = 8;                        // accelerator complex dies (each with its own L2)
// Cache policy of the K/V loads: nt (non-temporal).  Every cache byte is read exactly once per
// call, so keeping it in the caches only displaces other lines.
constexpr int kStreamOnce = 2;
static_assert(kBlocksPerSplit <= 64, "one block id per lane");

struct DecodeParams {
  const bf16* q;
  const bf16* kc;
  const bf16* vc;
  const int32_t* table;
  const int32_t* lens;
  bf16* o;
  float* lse;
  float* opart;  // [S][Hq][MS][D]
  float* mpart;  // [S][Hq][MS]
  float* lpart;  // [S][Hq][MS]
  int Hq, Hkv, group, max_blocks, max_tokens, MS, units;
  int num_blocks;  // blocks in the pool: ids outside [0, num_blocks) are never dereferenced
  int split;  // tokens per key range: kSplit or kLongSplit
  float sl2;
};

template <int D>
struct DGeo {
  static constexpr int RB = D * 2;              // bytes of one token's head row
  static constexpr int CPR = RB / 16;           // 16-byte chunks per row
  static constexpr int VTILE = kBS * RB;        // bytes of one block's V for one kv head
  static constexpr int NDMA = VTILE / 1024;     // 1 KB direct loads per block
  static constexpr int RPI = 1024 / RB;         // rows per direct load
  static constexpr int KC = D / 32;             // 16x16x32 MFMAs of the score contraction
  static constexpr int NB = D / 16;             // 16-dim output blocks
  // V chunk swizzle: the 16 rows x 32 bytes of one transposing read hit every bank group
  // exactly twice.
  __device__ static int swz(int row) { return D == 128 ? 2 * (row & 7) : 2 * ((row >> 1) & 3); }
  // K chunk swizzle: 16 consecutive rows read at one logical chunk hit 16 distinct bank groups.
  __device__ static int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
};

// Scalar state of one block: its buffer resources for K and V.
struct BlockRes {
  __amdgpu_buffer_rsrc_t k, v;
};

template <int D>
__device__ __forceinline__ BlockRes block_res(const DecodeParams& p, int bid, int valid_rows,
                                              int row_bytes) {
  const size_t base = (size_t)bid * kBS * p.Hkv * D;
  const int bytes = valid_rows * row_bytes;  // 0 for a block past the range
  BlockRes r;
  r.k = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(p.kc + base), (short)0, bytes,
                                          kBufferFlags);
  r.v = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(p.vc + base), (short)0, bytes,
                                          kBufferFlags);
  return r;
}

// Issue one block's loads: K into LDS stage `ks`, V into LDS stage `vs`, full rows per load.
template <int D>
__device__ __forceinline__ void issue_block(lds_t* ks, lds_t* vs, const BlockRes& r,
                                            const int (&koff)[DGeo<D>::NDMA],
                                            const int (&voff)[DGeo<D>::NDMA]) {
  using G = DGeo<D>;
#pragma unroll
  for (int t = 0; t < G::NDMA; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.k, ks + t * 1024, 16, koff[t], 0, 0, kStreamOnce);
#pragma unroll
  for (int t = 0; t < G::NDMA; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.v, vs + t * 1024, 16, voff[t], 0, 0, kStreamOnce);
}

// lgkmcnt(0): every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// vmcnt(n): wait until at most n vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

template <int D>
__global__ void __launch_bounds__(64) decode_split_kernel(DecodeParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer resources exist only for the GPU target
  using G = DGeo<D>;
  __shared__ __attribute__((aligned(1024))) char vs0[G::VTILE];
  __shared__ __attribute__((aligned(1024))) char vs1[G::VTILE];
  __shared__ __attribute__((aligned(1024))) char vs2[G::VTILE];
  __shared__ __attribute__((aligned(1024))) char vs3[G::VTILE];
  __shared__ __attribute__((aligned(1024))) char ks0[G::VTILE];
  __shared__ __attribute__((aligned(1024))) char ks1[G::VTILE];
  __shared__ __attribute__((aligned(1024))) char ks2[G::VTILE];
  __shared__ __attribute__((aligned(1024))) char ks3[G::VTILE];
  lds_t* const VS[kStages] = {(lds_t*)vs0, (lds_t*)vs1, (lds_t*)vs2, (lds_t*)vs3};
  lds_t* const KS[kStages] = {(lds_t*)ks0, (lds_t*)ks1, (lds_t*)ks2, (lds_t*)ks3};
  constexpr int kLoadsPerBlock = 2 * G::NDMA;

  const int lane = threadIdx.x;
  // Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Work unit u = one key range
  // of one sequence (b * MS + sp); its Hkv waves (one per kv head) take consecutive slots of one
  // XCD, so that XCD streams whole physical blocks ([16][Hkv][d] contiguous) while units go
  // round-robin over the XCDs (every XCD gets a share of every sequence).
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int g = slot % p.Hkv;
  const int u = (slot / p.Hkv) * kXcds + xcd;
  if (u >= p.units) return;
  const int b = u / p.MS, sp = u - b * p.MS;
  const int L = min(max(p.lens[b], 0), p.max_tokens);
  const int tok_begin = sp * p.split;
  if (tok_begin >= L) return;
  const int tok_end = min(L, tok_begin + p.split);
  const int blk_begin = tok_begin / kBS;
  const int n_blk = (tok_end - tok_begin + kBS - 1) / kBS;

  // Block ids of this range, one per lane (index prefetch into registers).
  const int my_bid = lane < n_blk ? p.table[(size_t)b * p.max_blocks + blk_begin + lane] : 0;

  const int row_bytes = p.Hkv * G::RB;
  const int col = lane & 15, grp = lane >> 4;
  // K and V: direct load t writes LDS rows RPI*t .. +RPI-1 (whole rows, so every load
  // instruction reads whole cache lines); lane -> (row, swizzled chunk).
  int koff[G::NDMA], voff[G::NDMA];
#pragma unroll
  for (int t = 0; t < G::NDMA; ++t) {
    const int row = t * G::RPI + lane / G::CPR;
    koff[t] = row * row_bytes + g * G::RB + (((lane % G::CPR) ^ G::swz_k(row)) * 16);
    voff[t] = row * row_bytes + g * G::RB + (((lane % G::CPR) ^ G::swz(row)) * 16);
  }
  // K fragment reads: for MFMA step c, lane holds token `col`, head dims 32c + 8*grp .. +7.
  int krd[G::KC];
#pragma unroll
  for (int c = 0; c < G::KC; ++c) krd[c] = col * G::RB + (((4 * c + grp) ^ G::swz_k(col)) << 4);
  // V^T fragment reads: group grp reads tokens 4*grp .. +3, dims 16n + 4*(s & 3) per source
  // lane s; the 16 lanes then hold 4 tokens of dims 16n .. 16n+15.
  int vrd[G::NB];
  {
    const int s = lane & 15;
    const int row = 4 * grp + (s >> 2);
#pragma unroll
    for (int n = 0; n < G::NB; ++n) {
      const int dim = 16 * n + 4 * (s & 3);
      vrd[n] = row * G::RB + (((dim >> 3) ^ G::swz(row)) << 4) + ((dim & 7) << 1);
    }
  }

  // Query fragments: B operand of S^T = K Q^T, column = head `col`, the same dims as K.
  const bool head_ok = col < p.group;
  const int qh = g * p.group + col;
  bf16x8 qf[G::KC];
#pragma unroll
  for (int c = 0; c < G::KC; ++c) {
    qf[c] = head_ok
                ? *reinterpret_cast<const bf16x8*>(p.q + ((size_t)b * p.Hq + qh) * D + 32 * c + 8 * grp)
                : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }

  // Scalar resources of block i of the range: empty past the end of the range, and empty for a
  // block id outside the pool (its keys and values then read as zeros; nothing outside the pool
  // is addressed).
  auto res_of = [&](int i) __attribute__((always_inline)) {
    int bid = __builtin_amdgcn_readlane(my_bid, min(i, n_blk - 1));
    int valid = i < n_blk ? min(kBS, tok_end - (tok_begin + i * kBS)) : 0;
    if ((unsigned)bid >= (unsigned)p.num_blocks) {
      bid = 0;
      valid = 0;
    }
    return block_res<D>(p, bid, valid, row_bytes);
  };

  f32x4 acc[G::NB];
#pragma unroll
  for (int n = 0; n < G::NB; ++n) acc[n] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;
  const float sl2 = p.sl2;

#pragma unroll
  for (int i = 0; i < kStages - 1; ++i) issue_block<D>(KS[i], VS[i], res_of(i), koff, voff);

  // Block i lives in stage i % kStages; issuing block i + kStages - 1 before computing block i
  // keeps kStages - 1 blocks of loads in flight.  Past the end the loads are empty (size 0) but
  // still issued, so the wait count below is the same on every step.
  auto step = [&](int i, auto stage) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage)::value;
    constexpr int NX = (ST + kStages - 1) % kStages;
    // Stage NX was read by the previous step.  The compiler does not see that the direct loads
    // write LDS, so it could move them above those reads: wait for every LDS read of this wave
    // and let nothing be scheduled across this point.
    wait_lds();
    __builtin_amdgcn_sched_barrier(0);
    issue_block<D>(KS[NX], VS[NX], res_of(i + kStages - 1), koff, voff);
    wait_vmem<(kStages - 1) * kLoadsPerBlock>();
    if (i >= n_blk) return;
    f32x4 s = f32x4{};
#pragma unroll
    for (int c = 0; c < G::KC; ++c)
      s = mfma16k32(*reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(KS[ST] + krd[c]),
                    qf[c], s);
    const int tok0 = tok_begin + i * kBS;
    if (tok0 + kBS > L) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (tok0 + 4 * grp + r >= L) s[r] = kNegInf;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = max_xor32(mx);
    const float mt = (mx == kNegInf) ? kNegInf : mx * sl2;
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float e[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float arg = fmaf(s[r], sl2, -m_use);
      if (s[r] == kNegInf) arg = kNegInf;  // exactly 0, also when the scale is 0
      e[r] = fast_exp2(arg);
    }
    l_run = fmaf(alpha, l_run, (e[0] + e[1]) + (e[2] + e[3]));
    u32x2 pk;
    pk[0] = pack_bf16x2(e[0], e[1]);
    pk[1] = pack_bf16x2(e[2], e[3]);
    const bf16x4 pf = __builtin_bit_cast(bf16x4, pk);
#pragma unroll
    for (int n = 0; n < G::NB; ++n) {
      const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(VS[ST] + vrd[n]));
      acc[n] = mfma16k16(__builtin_bit_cast(bf16x4, v), pf, acc[n] * alpha);
    }
  };
  for (int i = 0; i < n_blk; i += kStages) {
    step(i + 0, std::integral_constant<int, 0>{});
    step(i + 1, std::integral_constant<int, 1>{});
    step(i + 2, std::integral_constant<int, 2>{});
    step(i + 3, std::integral_constant<int, 3>{});
  }
  wait_vmem<0>();  // no direct load may still target this wave's LDS when it exits

  // Partial results of this range: lane (head col, grp) holds dims 16n + 4*grp + r.
  float lt = l_run + shfl_xor(l_run, 16);
  lt = add_xor32(lt);
  if (head_ok) {
    const size_t slot = ((size_t)b * p.Hq + qh) * p.MS + sp;
#pragma unroll
    for (int n = 0; n < G::NB; ++n)
      *reinterpret_cast<f32x4*>(p.opart + slot * D + 16 * n + 4 * grp) = acc[n];
    if (grp == 0) {
      p.mpart[slot] = m_run;
      p.lpart[slot] = lt;
    }
  }
#endif
}

// Merge the ranges of one (sequence, query head): M = max m_s, w_s = 2^(m_s - M),
// O = sum w_s O_s / sum w_s l_s, LSE = ln 2 * (M + log2 sum w_s l_s).  Lane s holds range s's
// statistics; the weighted sum over ranges is unrolled so that its loads overlap.
template <int D>
__global__ void __launch_bounds__(64) decode_merge_kernel(DecodeParams p) {
  constexpr int DPL = D / 64;  // dims per lane
  const int lane = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = min(max(p.lens[b], 0), p.max_tokens);
  const int n = (L + p.split - 1) / p.split;
  const size_t base = ((size_t)b * p.Hq + h) * p.MS;
  bf16* out = p.o + ((size_t)b * p.Hq + h) * D + lane * DPL;
  if (n == 0) {
#pragma unroll
    for (int j = 0; j < DPL; ++j) out[j] = static_cast<bf16>(0.f);
    if (p.lse != nullptr && lane == 0) p.lse[(size_t)b * p.Hq + h] = kNegInf;
    return;
  }
  float num[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) num[j] = 0.f;
  float M = kNegInf, den = 0.f;
  // Ranges are taken 64 at a time (one per lane); a sequence has at most MS of them.
  for (int s0 = 0; s0 < n; s0 += 64) {
    const int s = s0 + lane;
    const float ms = s < n ? p.mpart[base + s] : kNegInf;
    const float ls = s < n ? p.lpart[base + s] : 0.f;
    float mx = ms;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    const float M_new = fmaxf(M, mx);
    const float scale_old = fast_exp2(M - M_new);  // 0 on the first chunk (M = -inf)
    const float w = s < n ? fast_exp2(ms - M_new) : 0.f;
    float c = w * ls;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, 64);
    den = fmaf(den, scale_old, c);
#pragma unroll
    for (int j = 0; j < DPL; ++j) num[j] *= scale_old;
    const int cnt = min(64, n - s0);
    int t = 0;
    for (; t + 4 <= cnt; t += 4) {
      float x[4][DPL];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < DPL; ++j) x[u][j] = p.opart[(base + s0 + t + u) * D + lane * DPL + j];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wu = __shfl(w, t + u, 64);
#pragma unroll
        for (int j = 0; j < DPL; ++j) num[j] = fmaf(wu, x[u][j], num[j]);
      }
    }
    for (; t < cnt; ++t) {
      const float wu = __shfl(w, t, 64);
#pragma unroll
      for (int j = 0; j < DPL; ++j) num[j] = fmaf(wu, p.opart[(base + s0 + t) * D + lane * DPL + j], num[j]);
    }
    M = M_new;
  }
  const float inv = 1.f / den;
  if constexpr (DPL == 2) {
    *reinterpret_cast<uint32_t*>(out) = pack_bf16x2(num[0] * inv, num[1] * inv);
  } else {
    out[0] = static_cast<bf16>(num[0] * inv);
  }
  if (p.lse != nullptr && lane == 0)
    p.lse[(size_t)b * p.Hq + h] = (M + __log2f(den)) * kLn2;
}


template <int D>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  DecodeParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.kc = static_cast<const bf16*>(a.k_cache);
  p.vc = static_cast<const bf16*>(a.v_cache);
  p.table = a.block_table;
  p.lens = a.seq_lens;
  p.o = static_cast<bf16*>(a.o);
  p.lse = a.lse;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.max_blocks = a.max_blocks;
  p.max_tokens = a.max_blocks * a.block_size;
  p.num_blocks = a.num_blocks;
  // Range length: 1024 tokens when a full-length sequence still has at least 8 ranges and the
  // grid at least four rounds of waves (fewer partial results, and each wave's load ramp is paid
  // over twice the tokens), else 512: short contexts cut into 1024-token ranges leave a ragged
  // last round.  Measured, 512 -> 1024: 64 sequences U[512, 32768] 0.684 -> 0.667 ms, 32 such
  // 0.378 -> 0.372, 48 U[512, 16384] 0.311 -> 0.306, 256 U[512, 8192] 0.807 -> 0.784; but
  // 64 U[512, 4096] 0.127 -> 0.148 and 128 U[512, 4096] 0.218 -> 0.267, which keep 512.
  const long long long_ranges = (p.max_tokens + (long long)kLongSplit - 1) / kLongSplit;
  const long long long_waves = (long long)a.S * a.Hkv * long_ranges;
  p.split = (long_ranges >= kLongSplitMinRanges && long_waves >= kLongSplitMinWaves) ? kLongSplit
                                                                                     : kSplit;
  p.MS = decode_splits_of(a.max_blocks, a.block_size, p.split);
  const size_t slots = (size_t)a.S * a.Hq * p.MS;
  p.opart = static_cast<float*>(a.workspace);
  p.mpart = p.opart + slots * D;
  p.lpart = p.mpart + slots;
  p.sl2 = a.scale * kLog2e;
  p.units = a.S * p.MS;
  const long long grid_slots = (long long)((p.units + kXcds - 1) / kXcds) * a.Hkv;
  hipLaunchKernelGGL(decode_split_kernel<D>, dim3((unsigned)(grid_slots * kXcds)), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(a.Hq, a.S), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.d == 128 ? launch<128>(a, stream) : launch<64>(a, stream);
}

// ---------------------------------------------------------------------------------------------
// The decode without a caller workspace: the split partials go to a static device array of
// kDecodeScratchBytes, one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (in host code it is only a stand-in for the symbol): the device
// address of each GPU's copy is looked up once per device with hipGetSymbolAddress, with that
// device current, and that address is the workspace the kernels get.  Every partial the merge
// reads is written earlier in the same call, so nothing needs clearing.  Calls that overlap on
// one GPU share the array and race.
namespace {

static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void* scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

}  // namespace

hipError_t launch_paged_decode_noalloc(DecodeArgs a, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (stream != nullptr) {  // the scratch copy used is the current device's
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    if (sd != dev) return hipErrorInvalidDevice;
  }
  std::call_once(scratch_once[dev], [dev] {
    void* ptr = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (scratch_err[dev] != hipSuccess) return scratch_err[dev];
  if (decode_workspace_bytes(a.S, a.Hq, a.d, a.max_blocks, a.block_size) > kDecodeScratchBytes)
    return hipErrorInvalidValue;  // the entry point rejects these sizes before any HIP call
  a.workspace = scratch_ptr[dev];
  return launch_paged_decode(a, stream);
}

}  // namespace fa
