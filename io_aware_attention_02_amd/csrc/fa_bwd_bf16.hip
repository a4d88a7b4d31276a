// fa_bwd_bf16.hip -- attention backward with recomputation, bf16 storage, fp32 accumulation.
//
// The forward keeps only O and the per-row log-sum-exp; the backward recomputes the
// probabilities from them instead of storing the N x N matrix ("Gemini 3 Flash的注意力内核重写",
// §4 on recomputation: keep each row's maximum and normaliser, rebuild the scores when the
// gradients are needed).  With P = exp(S - LSE) (S = scale * Q K^T) and dO the output gradient:
//     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),   D_i = sum_j P_ij dP_ij = dO_i . O_i,
//     dQ = scale * dS K,   dK = scale * dS^T Q
// (the derivative of the softmax, with D the row-wise dot product the softmax Jacobian needs).
//
// Three kernels, every one deterministic (no atomics):
//  * bwd_pre_kernel   D_i = dO_i . O_i in fp32 for every row (0 for padding rows) and the LSE in
//                     base 2 (+inf for padding rows).
//  * bwd_dq_kernel    query-stationary, laid out like the forward: a wave owns 32 query rows,
//                     K and V tiles of 64 keys stream through LDS; S^T = K Q^T and dP^T = V dO^T
//                     on the matrix cores, dS^T in registers, dQ^T += K^T dS^T with K^T read by
//                     the transposing LDS read.
//  * bwd_dkdv_kernel  key-stationary: the workgroup's 128 K and V rows stay in LDS, query tiles
//                     of 64 rows of Q and dO (every query head of the kv head's group) stream
//                     through LDS; each wave runs S = Q K^T, dP = dO V^T, P, dS,
//                     dV^T += dO^T P and dK^T += Q^T dS for its 32 keys and 32 of the rows.
//                     Summing the group's heads inside the kernel keeps grouped-query dK/dV
//                     free of atomics.
// Every probability is rebuilt from the stored LSE as exp2(s * scale * log2 e - LSE * log2 e);
// padding rows get LSE = +inf here so that their probabilities are exactly 0.
#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tiles.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kNWb = 4;                 // waves per workgroup in both main kernels
constexpr int kXcdsB = 8;               // accelerator complex dies (each with its own L2)
constexpr float kPosInf = __builtin_huge_valf();

struct BwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const float* lse;
  const bf16* dout;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  float* dvec;  // D [B, H, N]
  float* lse2;  // LSE * log2 e [B, H, N] (+inf for padding rows)
  const int32_t* seq_lens;
  int B, H, group, Hkv, N, n_t, total;
  float scale, sl2;
};

__device__ __forceinline__ int valid_len(const BwdParams& p, int b) {
  return p.seq_lens != nullptr ? min(max(p.seq_lens[b], 0), p.N) : p.N;
}

// ---------------------------------------------------------------------------------------------
// D_i = dO_i . O_i: CPR lanes per row, 8 elements per lane, reduced across the lanes.
template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdParams p) {
  constexpr int CPR = D / 8;
  constexpr int RPB = 256 / CPR;  // rows per block
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / CPR;
  const int c = threadIdx.x % CPR;
  const long long rows = (long long)p.B * p.H * p.N;
  float acc = 0.f;
  int i = 0, L = 0;
  if (row < rows) {
    i = (int)(row % p.N);
    const int b = (int)(row / ((long long)p.H * p.N));
    L = valid_len(p, b);
    if (i < L) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(p.dout + row * D + 8 * c);
      const u32x4 o = *reinterpret_cast<const u32x4*>(p.o + row * D + 8 * c);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc = fmaf(__uint_as_float(a[t] << 16), __uint_as_float(o[t] << 16), acc);
        acc = fmaf(__uint_as_float(a[t] & 0xffff0000u), __uint_as_float(o[t] & 0xffff0000u), acc);
      }
    }
  }
#pragma unroll
  for (int m = CPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && c == 0) {
    p.dvec[row] = i < L ? acc : 0.f;
    p.lse2[row] = i < L ? p.lse[row] * kLog2e : kPosInf;
  }
}

// Every tile of the backward is read as rows (the A operand of a score product) and, apart
// from V in the dQ kernel, also transposed (the A operand of a gradient product), so all of
// them are stored with the two-way swizzle Geo::swz_b.  Per-lane offsets of the direct loads:
template <int D, int NW>
__device__ __forceinline__ void tile_offsets_b(int* off, int wave, int lane) {
  using G = Geo<D>;
  constexpr int NI_W = LoadGeo<D, NW>::NI_W;
#pragma unroll
  for (int t = 0; t < NI_W; ++t) {
    const int row = (wave * NI_W + t) * G::RPI + lane / G::CPR;
    off[t] = row * G::RB + (((lane % G::CPR) ^ G::swz_b(row)) << 4);
  }
}

// Row reads: row lane & 31, logical chunk 2c + (lane >> 5) (the layout of FragAddr::k).
template <int D>
__device__ __forceinline__ FragAddr<D> frag_addr_b(int lane) {
  using G = Geo<D>;
  FragAddr<D> a;
  const int c32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int c = 0; c < G::KC; ++c) a.k[c] = c32 * G::RB + (((2 * c + hh) ^ G::swz_b(c32)) << 4);
#pragma unroll
  for (int n = 0; n < G::NB; ++n) a.v[n] = 0;  // unused
  return a;
}

// Transposing reads: for 32-dim output block n, rows key and key + 8 of a 16-row chunk (the
// chunk base is added by the caller as 16 * jj rows; the swizzle of row 16 jj + r equals that
// of row r).
template <int D>
struct TrAddr {
  int lo[D / 32];
  int hi[D / 32];
};

template <int D>
__device__ __forceinline__ TrAddr<D> tr_addr_b(int lane) {
  using G = Geo<D>;
  TrAddr<D> a;
  const int grp = lane >> 4, s = lane & 15;
  const int key = 4 * (grp >> 1) + (s >> 2);
#pragma unroll
  for (int n = 0; n < G::NB; ++n) {
    const int dim = n * 32 + 16 * (grp & 1) + 4 * (s & 3);
    a.lo[n] = key * G::RB + (((dim >> 3) ^ G::swz_b(key)) << 4) + ((dim & 7) << 1);
    a.hi[n] = (key + 8) * G::RB + (((dim >> 3) ^ G::swz_b(key + 8)) << 4) + ((dim & 7) << 1);
  }
  return a;
}

// A^T fragment (32 dims of block n x 16 rows of chunk jj) of a tile.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const lds_t* tile, const TrAddr<D>& ta, int n, int jj) {
  using G = Geo<D>;
  const lds_t* base = tile + jj * 16 * G::RB;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + ta.lo[n]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + ta.hi[n]));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One 32-row block of a score product: s = rows[0..31] . bf over the head dimension (rows of a
// tile, B operand in registers), reads kAheadK fragments ahead of their MFMAs.
template <int D>
__device__ __forceinline__ void scores_block(f32x16& s, const lds_t* rows, const FragAddr<D>& fa,
                                             const bf16x8 (&bf)[D / 16]) {
  using G = Geo<D>;
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  s = f32x16{};
#pragma unroll
  for (int c = 0; c < G::KC; ++c)
    s = mfma32(*reinterpret_cast<const lds_bf16x8*>(rows + fa.k[c]), bf[c], s);
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kAheadK, 0);
#pragma unroll
  for (int i = 0; i < G::KC - kAheadK; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, kAheadK, 0);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
}

// Work unit = (batch, kv head): every workgroup of a unit reads the same K/V (dQ) or the same
// Q/dO of the group (dK/dV), so a unit's workgroups run on one XCD (shared L2); units are
// spread x, x+8, ... when they divide evenly so every XCD holds the same mix of lengths.
__device__ __forceinline__ void unit_of(const BwdParams& p, int per_unit, int& unit, int& rem) {
  const int lam = xcd_remap(blockIdx.x, p.total);
  const int units = p.total / per_unit;
  unit = lam / per_unit;
  rem = lam - unit * per_unit;
  if (units % kXcdsB == 0) unit = (unit % (units / kXcdsB)) * kXcdsB + unit / (units / kXcdsB);
}

// ---------------------------------------------------------------------------------------------
// dQ: one workgroup per (batch, query head, 128 query rows); waves own 32 rows each.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * kNWb) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_kernel(BwdParams p) {
  using G = Geo<D>;
  constexpr int NW = kNWb;
  constexpr int kBM = NW * kWQ;
  constexpr int NI_W = LoadGeo<D, NW>::NI_W;
  __shared__ __attribute__((aligned(1024))) char k0s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[G::TILE];
  lds_t* const K0 = (lds_t*)k0s;
  lds_t* const K1 = (lds_t*)k1s;
  lds_t* const V0 = (lds_t*)v0s;
  lds_t* const V1 = (lds_t*)v1s;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, hh = lane >> 5;
  int unit, rem;
  unit_of(p, p.group * p.n_t, unit, rem);
  const int b = unit / p.Hkv, g = unit - b * p.Hkv;
  // The group's query heads take consecutive slots for each query tile (same K/V rows side by
  // side, every head's heaviest tiles first).
  int qt = rem / p.group;
  const int hi = rem - qt * p.group;
  if (CAUSAL) qt = p.n_t - 1 - qt;  // heaviest query tiles first
  const int N = p.N, h = g * p.group + hi;
  const int bh = b * p.H + h;
  const int L = valid_len(p, b);
  const int q0 = qt * kBM;
  bf16* dQg = p.dq + (size_t)bh * N * D;
  if (q0 >= L) {  // padding rows only: dQ = 0
    const int rows = min(kBM, N - q0);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int i = tid; i < rows * G::CPR; i += 64 * NW)
      *reinterpret_cast<u32x4*>(dQg + (size_t)q0 * D + i * 8) = zero;
    return;
  }
  const bf16* Qg = p.q + (size_t)bh * N * D;
  const bf16* dOg = p.dout + (size_t)bh * N * D;
  const bf16* Kg = p.k + (size_t)(b * p.Hkv + g) * N * D;
  const bf16* Vg = p.v + (size_t)(b * p.Hkv + g) * N * D;

  const int kv_end = CAUSAL ? min(L, q0 + kBM) : L;
  const int n_kt = (kv_end + kBN - 1) / kBN;
  const int qw0 = q0 + wave * kWQ;
  const int qrow = qw0 + c32;
  const int n_kw = CAUSAL ? min(n_kt, (min(L, qw0 + kWQ) + kBN - 1) / kBN) : n_kt;
  const float sl2 = p.sl2;
  int off[NI_W];
  tile_offsets_b<D, NW>(off, wave, lane);
  load_tile<D, NW>(K0, Kg, 0, L, off, wave);
  load_tile<D, NW>(V0, Vg, 0, L, off, wave);

  // Q^T and dO^T fragments (B operands), zero for rows outside the valid length; the row's
  // LSE in base 2 (+inf for padding rows: probabilities exactly 0) and D.
  const bool valid = qrow < L;
  bf16x8 qf[G::KC], of[G::KC];
#pragma unroll
  for (int c = 0; c < G::KC; ++c) {
    const size_t at = (size_t)qrow * D + c * 16 + hh * 8;
    const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    qf[c] = valid ? *reinterpret_cast<const bf16x8*>(Qg + at) : zero;
    of[c] = valid ? *reinterpret_cast<const bf16x8*>(dOg + at) : zero;
  }
  const float lse2 = valid ? p.lse[(size_t)bh * N + qrow] * kLog2e : kPosInf;
  const float drow = valid ? p.dvec[(size_t)bh * N + qrow] : 0.f;
  const FragAddr<D> fa = frag_addr_b<D>(lane);
  const TrAddr<D> ta = tr_addr_b<D>(lane);

  f32x16 acc[G::NB];
#pragma unroll
  for (int n = 0; n < G::NB; ++n) acc[n] = f32x16{};
  f32x16 sS[2], sP[2];

  auto tile = [&](const lds_t* Kc, const lds_t* Vc, int key0, auto masked) __attribute__((always_inline)) {
    constexpr bool M = decltype(masked)::value;
    scores<D>(sS, Kc, fa, qf);
    scores<D>(sP, Vc, fa, of);
    if constexpr (M) mask_scores<CAUSAL>(sS, key0, L, qrow, hh);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float e[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float x = sS[jj >> 1][8 * (jj & 1) + t];
        float arg = fmaf(x, sl2, -lse2);
        if (M && x == kNegInf) arg = kNegInf;  // exactly 0, also when the scale is 0
        e[t] = fast_exp2(arg) * (sP[jj >> 1][8 * (jj & 1) + t] - drow);
      }
      const bf16x8 dsf = pack_bf16x8(e);
#pragma unroll
      for (int n = 0; n < G::NB; ++n) acc[n] = mfma32(tr_frag<D>(Kc, ta, n, jj), dsf, acc[n]);
    }
  };
  const int n_main = CAUSAL ? min(q0, L) / kBN : L / kBN;
  auto iter = [&](int j, auto parity, auto masked) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(parity)::value;
    lds_t* const Kc = ODD ? K1 : K0;
    lds_t* const Vc = ODD ? V1 : V0;
    lds_t* const Kn = ODD ? K0 : K1;
    lds_t* const Vn = ODD ? V0 : V1;
    if (j + 1 < n_kt) {
      load_tile<D, NW>(Kn, Kg, (j + 1) * kBN, L, off, wave);
      load_tile<D, NW>(Vn, Vg, (j + 1) * kBN, L, off, wave);
    }
    if (j < n_kw) tile(Kc, Vc, j * kBN, masked);
    wait_loads();
    __syncthreads();
  };
  wait_loads();
  __syncthreads();
  int j = 0;
  for (; j + 1 < n_main; j += 2) {
    iter(j, std::false_type{}, std::false_type{});
    iter(j + 1, std::true_type{}, std::false_type{});
  }
  for (; j < n_kt; ++j) {
    if (j & 1) iter(j, std::true_type{}, std::true_type{});
    else iter(j, std::false_type{}, std::true_type{});
  }

  if (qrow < N) {
#pragma unroll
    for (int n = 0; n < G::NB; ++n) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[n][4 * r4 + 0] * p.scale, acc[n][4 * r4 + 1] * p.scale);
        w[1] = pack_bf16x2(acc[n][4 * r4 + 2] * p.scale, acc[n][4 * r4 + 3] * p.scale);
        *reinterpret_cast<u32x2*>(dQg + (size_t)qrow * D + n * 32 + 8 * r4 + 4 * hh) = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dK, dV: one workgroup per (batch, kv head, 128 keys) of 8 waves.  The workgroup's K and V rows
// stay in LDS for the whole kernel (key-stationary: they are loaded once).  Wave w owns the 32
// keys of slice s = w & 3 and the rows 32 r .. 32 r + 31 (r = w >> 2) of every 64-row query
// tile, and runs all four products for that 32 x 32 block itself: S = Q K^T and dP = dO V^T
// (both operands read from LDS), P = exp2(S - LSE), dS = P o (dP - D), dV^T += dO^T P and
// dK^T += Q^T dS (the transposed operands by transposing LDS reads).  Nothing passes between
// waves inside the loop: the two waves of a SIMD (w and w + 4: the same keys, different rows)
// meet only at the tile barrier.  Their partial dK and dV are added once, at the end, through
// LDS, always wave w + 4's into wave w's: the sum order is fixed and the result deterministic.
//
// Query tiles of 64 rows (every query head of the group in turn: grouped-query sums need no
// atomics) are double-buffered in LDS with their LSE and D rows: tile t + 1 loads while tile t
// is computed, and one workgroup barrier per tile orders the buffer reuse.
constexpr int kNWkv = 8;
constexpr int kAheadKV = 2;  // fragment pairs read ahead of their MFMA in the score products

// Row statistics of a query tile (base-2 LSE or D, 64 fp32) straight into LDS, rows at or past
// the valid length reading 0: with zero Q and dO rows there, P = 1 and dP = D = 0, so such
// rows add exactly nothing to dK and dV.
__device__ __forceinline__ void load_stats(lds_t* dst, const float* rowbase, int row0, int L,
                                           int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int bytes = __builtin_amdgcn_readfirstlane(min(max(L - row0, 0), 64) * 4);  // one tile
  const uintptr_t base = reinterpret_cast<uintptr_t>(rowbase + row0);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uintptr_t)hi << 32) | lo), (short)0, bytes, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 4, lane * 4, 0, 0, 0);
#endif
}

// Hides the value's known bits from the compiler.  Applied once to the per-lane LDS offsets:
// an offset whose bits the compiler cannot see is added to an array's base address with an
// add that the fragment read absorbs into its 16-bit immediate offset, so one register serves
// every array below 64 KB; with the bits known, it ORs each array's base into a register of
// its own (one set per tile buffer, more than the registers hold).
__device__ __forceinline__ int hide_bits(int x) {
  asm("" : "+v"(x));
  return x;
}

// One 32 x 32 block of a score product with both operands in LDS: s = A[32 rows] . B[32 rows]
// over the head dimension (A rows give the output rows, B rows its columns), the fragment pairs
// read kAheadKV MFMAs ahead.  ao[c], bo[c]: lane offsets of the 16-dim step c in A and B.
template <int D>
__device__ __forceinline__ void scores_lds(f32x16& s, const lds_t* a, const int* ao,
                                           const lds_t* b, const int* bo) {
  using G = Geo<D>;
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  s = f32x16{};
#pragma unroll
  for (int c = 0; c < G::KC; ++c)
    s = mfma32(*reinterpret_cast<const lds_bf16x8*>(a + ao[c]),
               *reinterpret_cast<const lds_bf16x8*>(b + bo[c]), s);
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kAheadKV, 0);
#pragma unroll
  for (int i = 0; i < G::KC - kAheadKV; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, kAheadKV, 0);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * kNWkv) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_kernel(BwdParams p) {
  using G = Geo<D>;
  constexpr int NW = kNWkv;
  constexpr int kBK = 4 * kWQ;  // keys per workgroup
  constexpr int NI_W = LoadGeo<D, NW>::NI_W;
  static_assert(kBK == 2 * kBN, "the workgroup's keys are two LDS tiles");
  // The two query-tile buffers are separate arrays, always named statically (the loop below is
  // unrolled by two): the compiler then sees that the fragment reads of one buffer cannot alias
  // the direct loads in flight into the other, and puts no wait for those loads before them.
  __shared__ __attribute__((aligned(G::TILE))) char q0s[G::TILE];
  __shared__ __attribute__((aligned(G::TILE))) char q1s[G::TILE];
  __shared__ __attribute__((aligned(G::TILE))) char o0s[G::TILE];
  __shared__ __attribute__((aligned(G::TILE))) char o1s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char ks[2][G::TILE];  // K rows k0 .. k0 + 127
  __shared__ __attribute__((aligned(1024))) char vs[2][G::TILE];  // V rows
  __shared__ __attribute__((aligned(16))) float l0s[kBN];  // LSE (base 2) of the rows
  __shared__ __attribute__((aligned(16))) float l1s[kBN];
  __shared__ __attribute__((aligned(16))) float d0s[kBN];  // D of the rows
  __shared__ __attribute__((aligned(16))) float d1s[kBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, hh = lane >> 5;
  const int slice = wave & 3;
  const int rh = __builtin_amdgcn_readfirstlane(wave >> 2);  // which 32 rows of each query tile
  int unit, kt;
  unit_of(p, p.n_t, unit, kt);
  const int b = unit / p.Hkv, g = unit - b * p.Hkv;
  const int N = p.N;
  const int L = valid_len(p, b);
  const int k0 = kt * kBK;
  bf16* dKg = p.dk + (size_t)(b * p.Hkv + g) * N * D;
  bf16* dVg = p.dv + (size_t)(b * p.Hkv + g) * N * D;
  if (k0 >= L) {  // keys past the valid length: no query sees them, dK = dV = 0
    const int rows = min(kBK, N - k0);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int i = tid; i < rows * G::CPR; i += 64 * NW) {
      *reinterpret_cast<u32x4*>(dKg + (size_t)k0 * D + i * 8) = zero;
      *reinterpret_cast<u32x4*>(dVg + (size_t)k0 * D + i * 8) = zero;
    }
    return;
  }
  const int kw0 = k0 + slice * kWQ;
  const int key = kw0 + c32;  // this lane's key column
  const float sl2 = p.sl2;

  int off[NI_W];
  tile_offsets_b<D, NW>(off, wave, lane);
  // K and V rows of the workgroup (rows past the length read as zeros), loaded once.
  {
    const bf16* Kg = p.k + (size_t)(b * p.Hkv + g) * N * D;
    const bf16* Vg = p.v + (size_t)(b * p.Hkv + g) * N * D;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      load_tile<D, NW>((lds_t*)ks[t], Kg, k0 + t * kBN, L, off, wave);
      load_tile<D, NW>((lds_t*)vs[t], Vg, k0 + t * kBN, L, off, wave);
    }
  }

  // Query tiles: causal rows before the workgroup's first key never see it.
  const int qt0 = CAUSAL ? k0 / kBN : 0;
  const int n_q = (L + kBN - 1) / kBN - qt0;
  const int n_it = p.group * n_q;
  // Lane offsets of the fragment reads, the wave's place folded in: row reads of its 32 query
  // rows (qa) and of its 32 keys (ka), transposing reads of its two 16-row chunks (ta).
  int qa[G::KC], ka[G::KC];
  TrAddr<D> ta;
  {
    const FragAddr<D> fa = frag_addr_b<D>(lane);
    const TrAddr<D> t0 = tr_addr_b<D>(lane);
#pragma unroll
    for (int c = 0; c < G::KC; ++c) {
      qa[c] = hide_bits(fa.k[c] + rh * kWQ * G::RB);
      ka[c] = hide_bits(fa.k[c] + slice * kWQ * G::RB);
    }
#pragma unroll
    for (int n = 0; n < G::NB; ++n) {
      ta.lo[n] = hide_bits(t0.lo[n] + rh * kWQ * G::RB);
      ta.hi[n] = hide_bits(t0.hi[n] + rh * kWQ * G::RB);
    }
  }
  // Odd waves fetch the LSE row, even waves D (redundantly, so that every wave issues the same
  // number of loads per tile).
  auto issue = [&](int it, auto parity) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(parity)::value;
    const int hq = g * p.group + it / n_q;
    const int r0 = (qt0 + it % n_q) * kBN;
    const size_t hb = ((size_t)b * p.H + hq) * N;
    load_tile<D, NW>((lds_t*)(ODD ? q1s : q0s), p.q + hb * D, r0, L, off, wave);
    load_tile<D, NW>((lds_t*)(ODD ? o1s : o0s), p.dout + hb * D, r0, L, off, wave);
    if (wave & 1) load_stats((lds_t*)(ODD ? l1s : l0s), p.lse2 + hb, r0, L, lane);
    else load_stats((lds_t*)(ODD ? d1s : d0s), p.dvec + hb, r0, L, lane);
  };

  f32x16 dk[G::NB], dv[G::NB];  // dK^T and dV^T of the wave's keys, over its rows
#pragma unroll
  for (int n = 0; n < G::NB; ++n) {
    dk[n] = f32x16{};
    dv[n] = f32x16{};
  }

  // This wave's 32 rows of the tile in buffer buf: S and dP, then P and dS for the two 16-row
  // chunks jj = 2 rh + j2 (a lane holds rows 16 jj + 4 hh + {0..3} and 16 jj + 8 + 4 hh +
  // {0..3} of its key's column), then dV^T += dO^T P and dK^T += Q^T dS.
  auto step = [&](auto parity, int q0t, auto masked) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(parity)::value;
    constexpr bool M = decltype(masked)::value;
    const lds_t* const Qb = (const lds_t*)(ODD ? q1s : q0s);
    const lds_t* const Ob = (const lds_t*)(ODD ? o1s : o0s);
    const float* const lvec = ODD ? l1s : l0s;
    const float* const dvec = ODD ? d1s : d0s;
    f32x16 sx, sp;
    scores_lds<D>(sx, Qb, qa, (const lds_t*)ks, ka);
    scores_lds<D>(sp, Ob, qa, (const lds_t*)vs, ka);
    bf16x8 pf[2], df[2];
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
      const int jj = 2 * rh + j2;
      const f32x4 la = *reinterpret_cast<const f32x4*>(&lvec[16 * jj + 4 * hh]);
      const f32x4 lb = *reinterpret_cast<const f32x4*>(&lvec[16 * jj + 8 + 4 * hh]);
      const f32x4 da = *reinterpret_cast<const f32x4*>(&dvec[16 * jj + 4 * hh]);
      const f32x4 db = *reinterpret_cast<const f32x4*>(&dvec[16 * jj + 8 + 4 * hh]);
      float e[8], ds[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float arg = fmaf(sx[8 * j2 + t], sl2, -(t < 4 ? la[t & 3] : lb[t & 3]));
        if constexpr (M) {
          const int qr = q0t + 16 * jj + 8 * (t >> 2) + 4 * hh + (t & 3);
          if (key >= L || (CAUSAL && key > qr)) arg = kNegInf;
        }
        e[t] = fast_exp2(arg);
        ds[t] = e[t] * (sp[8 * j2 + t] - (t < 4 ? da[t & 3] : db[t & 3]));
      }
      pf[j2] = pack_bf16x8(e);
      df[j2] = pack_bf16x8(ds);
    }
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {  // ta holds the wave's rows: chunk j2 of them is jj
#pragma unroll
      for (int n = 0; n < G::NB; ++n) dv[n] = mfma32(tr_frag<D>(Ob, ta, n, j2), pf[j2], dv[n]);
#pragma unroll
      for (int n = 0; n < G::NB; ++n) dk[n] = mfma32(tr_frag<D>(Qb, ta, n, j2), df[j2], dk[n]);
    }
  };

  // Tile it in buffer it & 1 (parity static): tile it + 1 loads into the other buffer, which
  // was last read before the previous barrier.
  auto iter = [&](int it, auto parity) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(parity)::value;
    if (it + 1 < n_it) issue(it + 1, std::integral_constant<bool, !ODD>{});
    const int q0t = (qt0 + it % n_q) * kBN;
    // A wave whose rows all come before its keys (causal) skips the tile's arithmetic.
    const bool active = !CAUSAL || q0t + 32 * rh + 31 >= kw0;
    const bool masked = (CAUSAL && q0t + 32 * rh < kw0 + kWQ - 1) || kw0 + kWQ > L;
    if (active) {
      if (masked) step(parity, q0t, std::true_type{});
      else step(parity, q0t, std::false_type{});
    }
    wait_loads();  // tile it + 1 has landed
    __syncthreads();
  };
  issue(0, std::false_type{});
  wait_loads();
  __syncthreads();
  for (int it = 0; it < n_it; it += 2) {
    iter(it, std::false_type{});
    if (it + 1 < n_it) iter(it + 1, std::true_type{});
  }

  // Wave w + 4 hands its partial sums to wave w through LDS (every tile buffer is free now: the
  // loop ended with a barrier).  dK^T of slices 0-1 in ks, 2-3 in vs; dV^T of slice 0, 1, 2, 3
  // in q0s, q1s, o0s, o1s.
  {
    constexpr int kAccB = 64 * G::NB * 16 * 4;  // one accumulator of one wave, in bytes
    static_assert(kAccB == G::TILE, "one wave's accumulator per tile buffer");
    char* const vslot = slice == 0 ? q0s : slice == 1 ? q1s : slice == 2 ? o0s : o1s;
    f32x4* const xk = reinterpret_cast<f32x4*>((slice < 2 ? ks[0] : vs[0]) + (slice & 1) * kAccB);
    f32x4* const xv = reinterpret_cast<f32x4*>(vslot);
    if (rh == 1) {
#pragma unroll
      for (int n = 0; n < G::NB; ++n)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          xk[(n * 4 + r4) * 64 + lane] = f32x4{dk[n][4 * r4], dk[n][4 * r4 + 1], dk[n][4 * r4 + 2], dk[n][4 * r4 + 3]};
          xv[(n * 4 + r4) * 64 + lane] = f32x4{dv[n][4 * r4], dv[n][4 * r4 + 1], dv[n][4 * r4 + 2], dv[n][4 * r4 + 3]};
        }
    }
    __syncthreads();
    if (rh == 1) return;
#pragma unroll
    for (int n = 0; n < G::NB; ++n)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 a = xk[(n * 4 + r4) * 64 + lane];
        const f32x4 c = xv[(n * 4 + r4) * 64 + lane];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          dk[n][4 * r4 + t] += a[t];
          dv[n][4 * r4 + t] += c[t];
        }
      }
  }

  if (key < N) {
#pragma unroll
    for (int n = 0; n < G::NB; ++n) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dk[n][4 * r4 + 0] * p.scale, dk[n][4 * r4 + 1] * p.scale);
        wk[1] = pack_bf16x2(dk[n][4 * r4 + 2] * p.scale, dk[n][4 * r4 + 3] * p.scale);
        wv[0] = pack_bf16x2(dv[n][4 * r4 + 0], dv[n][4 * r4 + 1]);
        wv[1] = pack_bf16x2(dv[n][4 * r4 + 2], dv[n][4 * r4 + 3]);
        *reinterpret_cast<u32x2*>(dKg + (size_t)key * D + n * 32 + 8 * r4 + 4 * hh) = wk;
        *reinterpret_cast<u32x2*>(dVg + (size_t)key * D + n * 32 + 8 * r4 + 4 * hh) = wv;
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.o = static_cast<const bf16*>(a.o);
  p.lse = a.lse;
  p.dout = static_cast<const bf16*>(a.dout);
  p.dq = static_cast<bf16*>(a.dq);
  p.dk = static_cast<bf16*>(a.dk);
  p.dv = static_cast<bf16*>(a.dv);
  p.dvec = static_cast<float*>(a.workspace);
  p.lse2 = p.dvec + bwd_stat_floats(a.B, a.H, a.N);
  p.seq_lens = a.seq_lens;
  p.B = a.B;
  p.H = a.H;
  p.group = a.H / a.Hkv;
  p.Hkv = a.Hkv;
  p.N = a.N;
  p.scale = a.scale;
  p.sl2 = a.scale * kLog2e;
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     stream, p);
  p.n_t = (a.N + kNWb * kWQ - 1) / (kNWb * kWQ);
  p.total = a.B * a.Hkv * p.n_t;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(p.total), dim3(64 * kNWkv), 0, stream, p);
  p.total = a.B * a.H * p.n_t;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(p.total), dim3(64 * kNWb), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
