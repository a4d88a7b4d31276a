// fa_tiles.h -- tile machinery shared by the attention kernels (forward and backward).
//
// A K- or V-like tile is BN rows of d bf16 staged in LDS by direct global -> LDS loads, with
// the 16-byte chunks of each row XOR-swizzled so that the matrix-core fragment reads are free
// of bank conflicts; the 32x32x16 bf16 MFMA consumes rows of the tile as its A operand (score
// products) or, through the transposing LDS read, columns of it (weighted sums).  Only kernel
// sources include this file.
#pragma once

#include "fa_device.h"

namespace fa {
namespace {

typedef __attribute__((address_space(3))) char lds_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

constexpr int kWQ = 32;                // query rows per wave
constexpr int kBN = 64;                // keys per tile
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3: 32-bit data format, raw

template <int D>
struct Geo {
  static constexpr int RB = D * 2;                 // bytes per K/V row
  static constexpr int CPR = RB / 16;              // 16-byte chunks per row
  static constexpr int TILE = kBN * RB;            // bytes per K or V tile
  static constexpr int NI = TILE / 1024;           // 1 KB direct loads per tile
  static constexpr int RPI = 1024 / RB;            // rows per direct load
  static constexpr int KC = D / 16;                // 16-dim steps of the score contraction
  static constexpr int NB = D / 32;                // 32-dim blocks of the output
  // Chunk swizzles (XOR on the 16-byte chunk index of a row).  K: 16 consecutive rows read at
  // one logical chunk hit 16 distinct bank groups.  V: the 8 rows x 64 bytes that one
  // transposing read touches cover every bank group exactly twice.
  __device__ static int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  __device__ static int swz_v(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
  // Both ways (a tile read as rows and transposed): the K swizzle's row bits with the two 2-bit
  // halves exchanged.  16 consecutive rows still map to 16 distinct bank groups, and the 4
  // rows of one transposing read land in 4 different groups of 4 (the K swizzle puts them in
  // the same 4 groups: a 4-way conflict).
  __device__ static int swz_b(int row) {
    const int m = D == 128 ? (row & 15) : ((row >> 1) & 7);
    return D == 128 ? ((m & 3) << 2) | (m >> 2) : ((m & 1) << 2) | (m >> 1);
  }
};

// Direct tile loads per wave for a workgroup of NW waves.
template <int D, int NW>
struct LoadGeo {
  static constexpr int NI_W = Geo<D>::NI / NW;
  static_assert(Geo<D>::NI % NW == 0, "tile loads split evenly over the waves");
};

// Per-lane byte offsets of this wave's direct loads inside a tile (row * RB + swizzled chunk).
template <int D, int NW, bool IS_V>
__device__ __forceinline__ void tile_offsets(int* off, int wave, int lane) {
  using G = Geo<D>;
  constexpr int NI_W = LoadGeo<D, NW>::NI_W;
#pragma unroll
  for (int t = 0; t < NI_W; ++t) {
    const int row = (wave * NI_W + t) * G::RPI + lane / G::CPR;
    const int chunk = (lane % G::CPR) ^ (IS_V ? G::swz_v(row) : G::swz_k(row));
    off[t] = row * G::RB + chunk * 16;
  }
}

// Direct global -> LDS copy of one K or V tile (rows key0 .. key0+BN-1) through a buffer
// resource whose base is the tile's first row and whose size ends at the valid length L or at
// the tile's end, whichever comes first: rows at or past L are out of range and arrive as zeros
// (their scores are masked, so they add exactly nothing), no load can leave the tensor, and the
// 32-bit size cannot overflow however long the sequence.
template <int D, int NW>
__device__ __forceinline__ void load_tile(lds_t* dst, const bf16* head, int key0, int L,
                                          const int* off, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer-resource type exists only for the GPU target
  using G = Geo<D>;
  constexpr int NI_W = LoadGeo<D, NW>::NI_W;
  // The tile's base and size are the same for every lane; readfirstlane states it so the
  // resource stays in scalar registers.
  const int bytes = __builtin_amdgcn_readfirstlane(min(max(L - key0, 0), kBN) * G::RB);
  const uintptr_t base = reinterpret_cast<uintptr_t>(head + (size_t)key0 * D);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uintptr_t)hi << 32) | lo), (short)0, bytes, kBufferFlags);
#pragma unroll
  for (int t = 0; t < NI_W; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst + (wave * NI_W + t) * 1024, 16, off[t],
                                             0, 0, 0);
#endif
}

__device__ __forceinline__ void wait_loads() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); lgkm and exp counters untouched
}

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding
// (vmcnt in bits 3:0 and 15:14), leaving the other counters untouched.
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

// Per-lane LDS byte offsets of the fragment reads, fixed for the whole kernel.
template <int D>
struct FragAddr {
  int k[D / 16];  // K row (lane & 31), logical chunk 2c + (lane >> 5), for every c
  int v[D / 32];  // V transposing read for output block n, keys 4*hh' + (s >> 2)
};

template <int D>
__device__ __forceinline__ FragAddr<D> frag_addr(int lane) {
  using G = Geo<D>;
  FragAddr<D> a;
  const int c32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int c = 0; c < G::KC; ++c) a.k[c] = c32 * G::RB + (((2 * c + hh) ^ G::swz_k(c32)) << 4);
  const int grp = lane >> 4, s = lane & 15;
  const int key = 4 * (grp >> 1) + (s >> 2);
#pragma unroll
  for (int n = 0; n < G::NB; ++n) {
    const int dim = n * 32 + 16 * (grp & 1) + 4 * (s & 3);
    a.v[n] = key * G::RB + (((dim >> 3) ^ G::swz_v(key)) << 4) + ((dim & 7) << 1);
  }
  return a;
}

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedValu = 0x002;
constexpr int kValuPerMfma = 8;  // vector instructions placed after each P V MFMA

// S^T (64 keys x 32 queries of this wave) = K_tile Q^T: 2*D/16 fragment reads and MFMAs.  The
// reads run kAheadK fragments ahead of the MFMAs that consume them, which hides the LDS
// latency without holding the whole tile's fragments in registers.
constexpr int kAheadK = 4;
template <int D>
__device__ __forceinline__ void scores(f32x16 (&s)[2], const lds_t* Kb, const FragAddr<D>& fa,
                                       const bf16x8 (&qf)[D / 16]) {
  using G = Geo<D>;
  constexpr int NM = 2 * G::KC;
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int c = 0; c < G::KC; ++c) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 kf = *reinterpret_cast<const lds_bf16x8*>(Kb + fa.k[c] + kb * 32 * G::RB);
      s[kb] = mfma32(kf, qf[c], s[kb]);
    }
  }
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kAheadK, 0);
#pragma unroll
  for (int i = 0; i < NM - kAheadK; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, kAheadK, 0);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
}

// Masks the scores a query row may not see: keys at or past L, and (causal) keys after it.
template <bool CAUSAL>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[2], int key0, int L, int qrow, int hh) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      const bool ok = key < L && (!CAUSAL || key <= qrow);
      if (!ok) s[kb][r] = kNegInf;
    }
}

}  // namespace
}  // namespace fa
