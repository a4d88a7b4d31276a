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
//  * bwd_pre_kernel   D_i = dO_i . O_i in fp32 for every row (0 for padding rows).
//  * bwd_dq_kernel    query-stationary, laid out like the forward: a wave owns 32 query rows,
//                     K and V tiles of 64 keys stream through LDS; S^T = K Q^T and dP^T = V dO^T
//                     on the matrix cores, dS^T in registers, dQ^T += K^T dS^T with K^T read by
//                     the transposing LDS read.
//  * bwd_dkdv_kernel  key-stationary: a wave owns 32 keys (K, V in registers), query tiles of 64
//                     rows of Q and dO (every query head of the kv head's group) stream through
//                     LDS; S = Q K^T and dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS.
//                     Summing the group's heads inside the kernel keeps grouped-query dK/dV free
//                     of atomics.
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
  if (row < rows && c == 0) p.dvec[row] = i < L ? acc : 0.f;
}

// Per-lane LDS byte offsets of the transposing reads of a tile stored with the K swizzle: for
// 32-dim output block n, rows key and key + 8 of a 16-row chunk (the chunk base is added by
// the caller as 16 * jj rows; the swizzle of row 16 jj + r equals that of row r).
template <int D>
struct TrAddr {
  int lo[D / 32];
  int hi[D / 32];
};

template <int D>
__device__ __forceinline__ TrAddr<D> tr_addr_k(int lane) {
  using G = Geo<D>;
  TrAddr<D> a;
  const int grp = lane >> 4, s = lane & 15;
  const int key = 4 * (grp >> 1) + (s >> 2);
#pragma unroll
  for (int n = 0; n < G::NB; ++n) {
    const int dim = n * 32 + 16 * (grp & 1) + 4 * (s & 3);
    a.lo[n] = key * G::RB + (((dim >> 3) ^ G::swz_k(key)) << 4) + ((dim & 7) << 1);
    a.hi[n] = (key + 8) * G::RB + (((dim >> 3) ^ G::swz_k(key + 8)) << 4) + ((dim & 7) << 1);
  }
  return a;
}

// A^T fragment (32 dims of block n x 16 rows of chunk jj) of a K-swizzled tile.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const lds_t* tile, const TrAddr<D>& ta, int n, int jj) {
  using G = Geo<D>;
  const lds_t* base = tile + jj * 16 * G::RB;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + ta.lo[n]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + ta.hi[n]));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One 32-row block of a score product: s = rows[0..31] . bf over the head dimension (rows of a
// K-swizzled tile, B operand in registers), reads kAheadK fragments ahead of their MFMAs.
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
  const int hi = rem / p.n_t;
  int qt = rem - hi * p.n_t;
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
  tile_offsets<D, NW, false>(off, wave, lane);
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
  const FragAddr<D> fa = frag_addr<D>(lane);
  const TrAddr<D> ta = tr_addr_k<D>(lane);

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
// dK, dV: one workgroup per (batch, kv head, 128 keys); waves own 32 keys each.  The loop runs
// over every query head of the group and every query tile of 64 rows that can see the keys.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * kNWb) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dkdv_kernel(BwdParams p) {
  using G = Geo<D>;
  constexpr int NW = kNWb;
  constexpr int kBK = NW * kWQ;  // keys per workgroup
  constexpr int NI_W = LoadGeo<D, NW>::NI_W;
  __shared__ __attribute__((aligned(1024))) char q0s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char q1s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char o0s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char o1s[G::TILE];
  __shared__ __attribute__((aligned(16))) float lvec[2][kBN];  // LSE (base 2) of the tile rows
  __shared__ __attribute__((aligned(16))) float dvec[2][kBN];  // D of the tile rows
  lds_t* const Q0 = (lds_t*)q0s;
  lds_t* const Q1 = (lds_t*)q1s;
  lds_t* const O0 = (lds_t*)o0s;
  lds_t* const O1 = (lds_t*)o1s;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, hh = lane >> 5;
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
  const bf16* Kg = p.k + (size_t)(b * p.Hkv + g) * N * D;
  const bf16* Vg = p.v + (size_t)(b * p.Hkv + g) * N * D;
  const int kw0 = k0 + wave * kWQ;
  const int key = kw0 + c32;  // this lane's key column
  const float sl2 = p.sl2;

  // K^T and V^T fragments (B operands of S = Q K^T and dP = dO V^T), zero past the length.
  bf16x8 kf[G::KC], vf[G::KC];
#pragma unroll
  for (int c = 0; c < G::KC; ++c) {
    const size_t at = (size_t)key * D + c * 16 + hh * 8;
    const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    kf[c] = key < L ? *reinterpret_cast<const bf16x8*>(Kg + at) : zero;
    vf[c] = key < L ? *reinterpret_cast<const bf16x8*>(Vg + at) : zero;
  }

  // Query tiles: causal rows before the workgroup's first key never see it.
  const int qt0 = CAUSAL ? k0 / kBN : 0;
  const int n_q = (L + kBN - 1) / kBN - qt0;
  const int n_it = p.group * n_q;
  int off[NI_W];
  tile_offsets<D, NW, false>(off, wave, lane);
  const FragAddr<D> fa = frag_addr<D>(lane);
  const TrAddr<D> ta = tr_addr_k<D>(lane);
  // Iteration it -> (query head of the group, query tile).
  auto head_of = [&](int it) __attribute__((always_inline)) { return g * p.group + it / n_q; };
  auto qrow0 = [&](int it) __attribute__((always_inline)) { return (qt0 + it % n_q) * kBN; };
  // Row statistics of a tile: each wave fills 16 of the 64 entries (+inf / 0 past the length).
  float l_next = kPosInf, d_next = 0.f;
  auto fetch_stats = [&](int it) __attribute__((always_inline)) {
    const int r = qrow0(it) + wave * 16 + (lane & 15);
    const size_t at = ((size_t)b * p.H + head_of(it)) * N + r;
    const bool ok = lane < 16 && r < L;
    l_next = ok ? p.lse[at] * kLog2e : kPosInf;
    d_next = ok ? p.dvec[at] : 0.f;
  };
  auto store_stats = [&](int buf) __attribute__((always_inline)) {
    if (lane < 16) {
      lvec[buf][wave * 16 + lane] = l_next;
      dvec[buf][wave * 16 + lane] = d_next;
    }
  };
  auto load_q = [&](int it, lds_t* Qd, lds_t* Od) __attribute__((always_inline)) {
    const size_t hb = ((size_t)b * p.H + head_of(it)) * N * D;
    load_tile<D, NW>(Qd, p.q + hb, qrow0(it), L, off, wave);
    load_tile<D, NW>(Od, p.dout + hb, qrow0(it), L, off, wave);
  };

  f32x16 dk[G::NB], dv[G::NB];
#pragma unroll
  for (int n = 0; n < G::NB; ++n) dk[n] = dv[n] = f32x16{};

  // One LDS tile of 64 query rows, in two halves of 32: S = Q K^T and dP = dO V^T for the
  // half (rows = queries, lane column = key), then per 16-row chunk P and dS and the dV^T, dK^T
  // updates.  Working in halves keeps only one score block of each product live.
  auto tile = [&](const lds_t* Qc, const lds_t* Oc, int buf, int q0t, auto masked) __attribute__((always_inline)) {
    constexpr bool M = decltype(masked)::value;
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      f32x16 sS, sP;
      scores_block<D>(sS, Qc + hq * 32 * G::RB, fa, kf);
      scores_block<D>(sP, Oc + hq * 32 * G::RB, fa, vf);
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        const int jj = 2 * hq + j2;
        // Rows of chunk jj held by this lane: 16 jj + 4 hh + {0..3} and 16 jj + 8 + 4 hh + {0..3}.
        const f32x4 la = *reinterpret_cast<const f32x4*>(&lvec[buf][16 * jj + 4 * hh]);
        const f32x4 lb = *reinterpret_cast<const f32x4*>(&lvec[buf][16 * jj + 8 + 4 * hh]);
        const f32x4 da = *reinterpret_cast<const f32x4*>(&dvec[buf][16 * jj + 4 * hh]);
        const f32x4 db = *reinterpret_cast<const f32x4*>(&dvec[buf][16 * jj + 8 + 4 * hh]);
        float pe[8], de[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float x = sS[8 * j2 + t];
          const float l2 = t < 4 ? la[t & 3] : lb[t & 3];
          const float dd = t < 4 ? da[t & 3] : db[t & 3];
          float arg = fmaf(x, sl2, -l2);
          if constexpr (M) {
            const int qr = q0t + 16 * jj + 8 * (t >> 2) + 4 * hh + (t & 3);
            if (key >= L || (CAUSAL && key > qr)) arg = kNegInf;
          }
          pe[t] = fast_exp2(arg);
          de[t] = pe[t] * (sP[8 * j2 + t] - dd);
        }
        const bf16x8 pf = pack_bf16x8(pe);
        const bf16x8 dsf = pack_bf16x8(de);
#pragma unroll
        for (int n = 0; n < G::NB; ++n) {
          dv[n] = mfma32(tr_frag<D>(Oc, ta, n, jj), pf, dv[n]);
          dk[n] = mfma32(tr_frag<D>(Qc, ta, n, jj), dsf, dk[n]);
        }
      }
    }
  };
  // A tile needs the mask when it straddles the causal diagonal of this workgroup's keys or
  // when some of those keys lie past the valid length; a wave whose keys all come after the
  // tile's last row skips it.
  auto iter = [&](int it, auto parity) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(parity)::value;
    lds_t* const Qc = ODD ? Q1 : Q0;
    lds_t* const Oc = ODD ? O1 : O0;
    lds_t* const Qn = ODD ? Q0 : Q1;
    lds_t* const On = ODD ? O0 : O1;
    constexpr int BUF = ODD ? 1 : 0;
    if (it + 1 < n_it) {
      load_q(it + 1, Qn, On);
      fetch_stats(it + 1);
    }
    const int q0t = qrow0(it);
    const bool masked = (CAUSAL && q0t < k0 + kBK - 1) || k0 + kBK > L;
    if (!CAUSAL || q0t + kBN - 1 >= kw0) {
      if (masked) tile(Qc, Oc, BUF, q0t, std::true_type{});
      else tile(Qc, Oc, BUF, q0t, std::false_type{});
    }
    if (it + 1 < n_it) store_stats(1 - BUF);
    wait_loads();
    __syncthreads();
  };
  load_q(0, Q0, O0);
  fetch_stats(0);
  store_stats(0);
  wait_loads();
  __syncthreads();
  int it = 0;
  for (; it + 1 < n_it; it += 2) {
    iter(it, std::false_type{});
    iter(it + 1, std::true_type{});
  }
  if (it < n_it) iter(it, std::false_type{});

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
        const size_t at = (size_t)key * D + n * 32 + 8 * r4 + 4 * hh;
        *reinterpret_cast<u32x2*>(dKg + at) = wk;
        *reinterpret_cast<u32x2*>(dVg + at) = wv;
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
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(p.total), dim3(64 * kNWb), 0, stream, p);
  p.total = a.B * a.H * p.n_t;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(p.total), dim3(64 * kNWb), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return ((size_t)B * H * N * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
