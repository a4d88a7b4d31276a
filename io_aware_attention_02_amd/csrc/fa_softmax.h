// fa_softmax.h -- the online-softmax step of the fused bf16 forward kernels (contiguous and
// paged): probabilities of a score tile and their weighted sum of V on the matrix cores.
// Only kernel sources include this file.
#pragma once

#include "fa_device.h"
#include "fa_tiles.h"

namespace fa {
namespace {

constexpr float kTau = 16.f;           // headroom of a fixed reference maximum (log2 units)
constexpr float kMaxProb = 65536.f;    // 2^kTau

__device__ __forceinline__ float tile_max(const f32x16 (&s)[2]) {
  float m0 = s[0][0], m1 = s[1][0];
#pragma unroll
  for (int r = 1; r < 16; ++r) {
    m0 = fmaxf(m0, s[0][r]);
    m1 = fmaxf(m1, s[1][r]);
  }
  return max_xor32(fmaxf(m0, m1));
}

// Probabilities of one 16-key chunk (jj) of the tile: exp2(s * sl2 - m), packed to bf16 in the
// k-slot order of the P^T operand; their sum is added to rs.  On masked tiles a masked score
// (-inf) gives exactly 0 even when the scale is 0 (where -inf * 0 would be NaN).
template <bool MASKED>
__device__ __forceinline__ bf16x8 chunk_probs(const f32x16 (&s)[2], int jj, float sl2, float m_use,
                                              float& rs) {
  float e[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float x = s[jj >> 1][8 * (jj & 1) + t];
    float arg = fmaf(x, sl2, -m_use);
    if (MASKED && x == kNegInf) arg = kNegInf;
    e[t] = fast_exp2(arg);
  }
  rs += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  return pack_bf16x8(e);
}

// Softmax and O^T (d x 32 queries) = alpha O^T + V_tile^T P^T, interleaved.  The MFMAs run
// chunk by chunk (16 keys) over the D/32 output blocks, each fed by two transposing V reads
// kAheadV MFMAs ahead.  While they run, the vector ALU rescales the output blocks not yet
// touched (alpha) and computes the next chunk's probabilities, so most of the softmax hides
// under the matrix work.  Returns this lane's part of the tile's row sum.
constexpr int kAheadV = 4;
template <int D, bool MASKED, bool RESCALE>
__device__ __forceinline__ float softmax_pv(f32x16 (&acc)[D / 32], const lds_t* Vb,
                                            const FragAddr<D>& fa, const f32x16 (&s)[2],
                                            float sl2, float m_use, float alpha) {
  using G = Geo<D>;
  constexpr int NM = 4 * G::NB;
  float rs = 0.f;
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 pf[4];
  pf[0] = chunk_probs<MASKED>(s, 0, sl2, m_use, rs);
  if (RESCALE) acc[0] *= alpha;
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
    for (int n = 0; n < G::NB; ++n) {
      const lds_t* p = Vb + fa.v[n] + jj * 16 * G::RB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * G::RB));
      const bf16x8 vf = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      if (RESCALE && jj == 0 && n + 1 < G::NB) acc[n + 1] *= alpha;
      acc[n] = mfma32(vf, pf[jj], acc[n]);
    }
    if (jj + 1 < 4) pf[jj + 1] = chunk_probs<MASKED>(s, jj + 1, sl2, m_use, rs);
  }
  // Schedule: the first reads, then per MFMA a few vector instructions and the next reads.
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kAheadV, 0);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, kValuPerMfma, 0);
    if (i + kAheadV < NM) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  return rs;
}

}  // namespace
}  // namespace fa
