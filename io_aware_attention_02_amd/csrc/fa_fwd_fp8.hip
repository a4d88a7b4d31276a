// fa_fwd_fp8.hip -- fused attention forward with FP8 (e4m3) Q, K, V on the gfx950 FP8 MFMA.
//
// The FP8 variant of the fused forward: Q, K and V arrive as e4m3 codes with one descale
// factor per tensor (the FP8 tensor-core attention the "GPU优化" tag page attributes to
// FlashAttention V3, excerpt "注意力计算的性能瓶颈").  Both products run on
// v_mfma_f32_32x32x64_f8f6f4 (64-deep contraction, fp32 accumulation): the scores S^T = K Q^T
// from the codes (the descale factors fold into the softmax scale), and O^T += V^T P^T with the
// probabilities rounded to e4m3.  The softmax is the online recurrence of "FlashAttention优化"
// §3.2.1 over blocks of 64 keys.  The probabilities exp(s - m) relative to a per-row reference m
// are multiplied by 64 before the rounding (small values stay out of the subnormals); the row
// sum uses them unrounded, and the output is multiplied by v_scale / sum at the end.  The first
// pass (FAST) fixes m after the first 128 keys at their maximum + 4 (log2 units), so later
// blocks need no row maximum and nothing is rescaled; a probability that would not fit e4m3
// becomes NaN in the conversion and sends the workgroup to the second pass (SAFE), in which m
// moves to a block's maximum whenever that maximum exceeds it by more than a factor 2^2
// (probabilities <= 4, 64 p <= 256).
//
// CDNA4 mapping:
//  * A wave owns 32 query rows, an LDS tile is 128 keys (two softmax blocks); workgroups of 8
//    waves (256 rows, one per CU) or 4 waves (128 rows) as in the bf16 forward.  K and V tiles
//    (128 x d bytes) go from global memory straight into LDS (buffer_load ... lds),
//    double-buffered, one barrier per tile.
//  * Operand layout of the FP8 MFMA (measured): lane l holds row l & 31 of A and column l & 31
//    of B, 32 bytes each; byte j of the lanes l >> 5 = h is the same contraction slot in A and
//    B.  Scores: A = K rows (32 keys), B = Q rows in registers, slot (h, j) = dimension
//    64 c + 32 h + j.  The accumulator holds one query per lane and, of a 32-key block, keys
//    8 (r >> 2) + 4 h + (r & 3) for r = 0..15.
//  * P V: the probabilities of two 32-key blocks, converted to e4m3 in accumulator order, are
//    directly the B operand (slot (h, j) = key 32 (j >> 4) + 8 ((j & 15) >> 2) + 4 h + (j & 3)).
//    The A operand V^T (32 dims x the same 64 keys) comes from ds_read_b64_tr_b8, the 8-bit
//    transposing LDS read: within each 16-lane group, output lane s gets byte s & 7 of the
//    8-byte row piece addressed by lane 2 b + (s >> 3), for b = 0..7.  Four such reads fill one
//    operand.
//  * The 16-byte chunks of the K and V rows in LDS are XOR-swizzled by key so that the row
//    reads (K) and the transposing reads (V) are free of bank conflicts.
#include "fa_device.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {
namespace {

typedef __attribute__((address_space(3))) char lds8_t;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kCUs8 = 256;
constexpr int kXcds8 = 8;
constexpr int kWQ8 = 32;               // query rows per wave
constexpr int kBN8 = 128;              // keys per tile
constexpr int kPScaleLog2 = 6;         // probabilities are rounded to e4m3 as 64 p
constexpr float kLagLog2 = 2.f;        // a row's reference moves when outgrown by more than 2^2
constexpr float kHeadLog2 = 4.f;       // FAST pass: fixed reference 2^4 above the first tile's maximum
constexpr int kBufFlags8 = 0x00020000; // buffer resource word 3: 32-bit data format, raw
constexpr int kSchedMfma8 = 0x008;     // instruction-group masks of sched_group_barrier
constexpr int kSchedDsRead8 = 0x100;
constexpr int kSchedValu8 = 0x002;
constexpr int kAhead8 = 2;             // score MFMAs whose K reads are in flight
constexpr int kAheadV8 = 2;            // P V MFMAs whose V reads are in flight

template <int D>
struct Geo8 {
  static constexpr int RB = D;                // bytes per row
  static constexpr int CPR = D / 16;          // 16-byte chunks per row
  static constexpr int TILE = kBN8 * RB;      // bytes per K or V tile
  static constexpr int NI = TILE / 1024;      // 1 KB direct loads per tile
  static constexpr int RPI = 1024 / RB;       // rows per direct load
  static constexpr int KC = D / 64;           // 64-deep steps of the score contraction
  static constexpr int NB = D / 32;           // 32-dim output blocks
  // K: 16 consecutive rows read at one logical chunk hit 16 distinct 16-byte bank groups.
  __device__ static int swz_k(int row) { return D == 128 ? (row >> 1) & 7 : (row >> 2) & 3; }
  // V: the 8 keys x 32 bytes of one half-wave transposing read hit 16 distinct bank groups.
  __device__ static int swz_v(int row) {
    return D == 128 ? 2 * ((row >> 1) & 1) + 4 * ((row >> 3) & 1) : 2 * ((row >> 3) & 1);
  }
};

struct Params8 {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  bf16* o;
  float* lse;
  const int32_t* seq_lens;
  int H, group, Hkv, N, n_qt, total;
  float sl2;      // scale * q_scale * k_scale * log2(e)
  float v_scale;  // descale of V
};

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  // e4m3 for both operands, no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four e4m3 bytes from four floats (round to nearest even), a first.  The first conversion
// writes the low half of the word and keeps the high half of its third operand, which the
// second overwrites; a's own bits serve, so the conversion can reuse a's register in place.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int D, int NW>
__device__ __forceinline__ void tile_offsets8(int* off, int wave, int lane, bool is_v) {
  using G = Geo8<D>;
  constexpr int NI_W = G::NI / NW;
#pragma unroll
  for (int t = 0; t < NI_W; ++t) {
    const int row = (wave * NI_W + t) * G::RPI + lane / G::CPR;
    const int chunk = (lane % G::CPR) ^ (is_v ? G::swz_v(row) : G::swz_k(row));
    off[t] = row * G::RB + chunk * 16;
  }
}

// Direct global -> LDS copy of one tile (rows key0 .. key0 + 127); rows at or past L read zero.
// The resource size stops at the tile's end, so it cannot overflow for long sequences.
template <int D, int NW>
__device__ __forceinline__ void load_tile8(lds8_t* dst, const uint8_t* head, int key0, int L,
                                           const int* off, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
  using G = Geo8<D>;
  constexpr int NI_W = G::NI / NW;
  const int bytes = __builtin_amdgcn_readfirstlane(min(max(L - key0, 0), kBN8) * G::RB);
  const uintptr_t base = reinterpret_cast<uintptr_t>(head + (size_t)key0 * D);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uintptr_t)hi << 32) | lo), (short)0, bytes, kBufFlags8);
#pragma unroll
  for (int t = 0; t < NI_W; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst + (wave * NI_W + t) * 1024, 16, off[t],
                                             0, 0, 0);
#endif
}

__device__ __forceinline__ void wait_loads8() { __builtin_amdgcn_s_waitcnt(0x0f70); }

template <int D, bool CAUSAL, int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_fp8_kernel(Params8 p) {
  using G = Geo8<D>;
  constexpr int kBM = NW * kWQ8;
  constexpr int kThreads = 64 * NW;
  constexpr int NI_W = G::NI / NW;
  __shared__ __attribute__((aligned(1024))) char k0s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[G::TILE];
  lds8_t* const K0 = (lds8_t*)k0s;
  lds8_t* const K1 = (lds8_t*)k1s;
  lds8_t* const V0 = (lds8_t*)v0s;
  lds8_t* const V1 = (lds8_t*)v1s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: kept in a scalar register
  const int c32 = lane & 31, hh = lane >> 5;

  // Work unit = (batch, kv head), remapped so its tiles share an XCD (as in the bf16 forward).
  const int lam = xcd_remap(blockIdx.x, p.total);
  const int per_unit = p.group * p.n_qt;
  const int units = p.total / per_unit;
  int unit = lam / per_unit;
  const int rem = lam - unit * per_unit;
  if (units % kXcds8 == 0) unit = (unit % (units / kXcds8)) * kXcds8 + unit / (units / kXcds8);
  const int b = unit / p.Hkv, g = unit - b * p.Hkv;
  // The group's query heads take consecutive slots for each query tile (same K/V rows side by
  // side, every head's heaviest tiles first).
  int qt = rem / p.group;
  const int hi = rem - qt * p.group;
  if (CAUSAL) qt = p.n_qt - 1 - qt;  // heaviest query tiles first
  const int N = p.N;
  const int h = g * p.group + hi;
  const int bh = b * p.H + h;
  const int L = p.seq_lens != nullptr ? min(max(p.seq_lens[b], 0), N) : N;

  const int q0 = qt * kBM;
  const uint8_t* Qg = p.q + (size_t)bh * N * D;
  const uint8_t* Kg = p.k + (size_t)(b * p.Hkv + g) * N * D;
  const uint8_t* Vg = p.v + (size_t)(b * p.Hkv + g) * N * D;
  bf16* Og = p.o + (size_t)bh * N * D;
  float* LSEg = p.lse + (size_t)bh * N;

  if (q0 >= L) {  // padding rows only: O = 0, LSE = -inf
    const int rows = min(kBM, N - q0);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int i = tid; i < rows * (D / 8); i += kThreads)
      *reinterpret_cast<u32x4*>(Og + (size_t)q0 * D + i * 8) = zero;
    for (int r = tid; r < rows; r += kThreads) LSEg[q0 + r] = kNegInf;
    return;
  }

  const int kv_end = CAUSAL ? min(L, q0 + kBM) : L;
  const int n_kt = (kv_end + kBN8 - 1) / kBN8;
  const int qw0 = q0 + wave * kWQ8;
  const int qrow = qw0 + c32;
  const int n_kw = qw0 >= L ? 0  // every row of this wave is padding
                 : CAUSAL ? min(n_kt, (min(L, qw0 + kWQ8) + kBN8 - 1) / kBN8) : n_kt;
  const float sl2 = p.sl2;
  int koff[NI_W], voff[NI_W];
  tile_offsets8<D, NW>(koff, wave, lane, false);
  tile_offsets8<D, NW>(voff, wave, lane, true);
  load_tile8<D, NW>(K0, Kg, 0, L, koff, wave);
  load_tile8<D, NW>(V0, Vg, 0, L, voff, wave);

  // Q fragments (B operand): 32 bytes per 64-deep step, zero for padding rows.
  i32x8 qf[G::KC];
#pragma unroll
  for (int c = 0; c < G::KC; ++c) {
    u32x4 lo = {0u, 0u, 0u, 0u}, hi4 = {0u, 0u, 0u, 0u};
    if (qrow < L) {
      const uint8_t* src = Qg + (size_t)qrow * D + 64 * c + 32 * hh;
      lo = *reinterpret_cast<const u32x4*>(src);
      hi4 = *reinterpret_cast<const u32x4*>(src + 16);
    }
    qf[c] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                  (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
  }
  // LDS byte offsets: K row reads (row c32 of a 32-key block, chunks 4c + 2h and 4c + 2h + 1)
  // and the V transposing reads (output block n; keys of read q and key chunk kc are added as
  // immediate row offsets, which leave the swizzle unchanged).
  int kaddr[G::KC][2];
#pragma unroll
  for (int c = 0; c < G::KC; ++c)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      kaddr[c][e] = c32 * G::RB + (((4 * c + 2 * hh + e) ^ G::swz_k(c32)) << 4);
  int vaddr[G::NB];
  {
    const int grp = lane >> 4, s = lane & 15;
    const int bb = s >> 1, odd = s & 1, hv = grp >> 1;
    const int key = 8 * (bb >> 2) + 4 * hv + (bb & 3);
#pragma unroll
    for (int n = 0; n < G::NB; ++n) {
      const int dim = 32 * n + 16 * (grp & 1) + 8 * odd;
      vaddr[n] = key * G::RB + (((dim >> 4) ^ G::swz_v(key)) << 4) + (dim & 15);
    }
  }

  f32x16 acc[G::NB];
#pragma unroll
  for (int n = 0; n < G::NB; ++n) acc[n] = f32x16{};
  float m_run = kNegInf;  // row reference (log2 units)
  float l_run = 0.f;      // this lane's share of the row sum, times 64
  float m_seen = kNegInf; // FAST pass: the row maximum over its first tile (log2 units)

  // The K/V loop runs in one of two passes.
  //  * SAFE: the lagging reference above on every block; each block needs its row maximum.
  //  * FAST (first try): the lagging reference on the first tile only, whose exact row maximum
  //    is kept; then the reference is fixed at that maximum + kHeadLog2 (O and l rescaled once)
  //    and later blocks compute no maximum.  Every probability is then at most 2^kHeadLog2
  //    below the row's largest one, and the row's largest is at least 2^-kHeadLog2.  A
  //    probability above 7.25 (64 p above 464) has no e4m3 code: the conversion returns NaN,
  //    which the FP8 MFMA carries into every accumulator element of that query, so one NaN test
  //    per lane after the loop finds it, and the workgroup recomputes in the SAFE pass.  On
  //    random inputs a row's maximum exceeds its first tile's by at most about 2^5.5 (16K keys),
  //    so the fallback is rare; inputs holding NaN take it too and give the SAFE result.
  enum { FIRST = 0, FAST = 1, SAFE = 2 };
  constexpr int NS = 2 * G::KC;  // score MFMAs of a 64-key block
  // K fragment (A operand) of 32-key block bl of 64-key block hk, 64-deep step c: two 16-byte
  // row reads.
  auto kfrag = [&](const lds8_t* Kc, int hk, int bl, int c) __attribute__((always_inline)) {
    const lds8_t* rb = Kc + (64 * hk + 32 * bl) * G::RB;
    const u32x4 a0 = *reinterpret_cast<const lds_u32x4*>(rb + kaddr[c][0]);
    const u32x4 a1 = *reinterpret_cast<const lds_u32x4*>(rb + kaddr[c][1]);
    return i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                 (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  };
  // V^T fragment (A operand of P V) of output block n and 64-key block hk: four transposing
  // reads of the keys 64 hk + 16 q ...
  auto vfrag = [&](const lds8_t* Vc, int hk, int n) __attribute__((always_inline)) {
    i32x8 vf;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_i32x2*)(Vc + vaddr[n] + (64 * hk + 16 * q) * G::RB));
      vf[2 * q] = r2[0];
      vf[2 * q + 1] = r2[1];
    }
    return vf;
  };
  // Scores of keys 64 hk .. 64 hk + 63 (two 32-key blocks).
  auto score_mfmas = [&](f32x16 (&sc)[2], const lds8_t* Kc, int hk) __attribute__((always_inline)) {
#pragma unroll
    for (int bl = 0; bl < 2; ++bl) {
      sc[bl] = f32x16{};
#pragma unroll
      for (int c = 0; c < G::KC; ++c) sc[bl] = mfma8(kfrag(Kc, hk, bl, c), qf[c], sc[bl]);
    }
  };
  // Probabilities exp2(s sl2 - bias) as e4m3 in k-slot order (the B operand of P V); returns
  // their unrounded sum.  On masked tiles a masked score (-inf) gives exactly 0, also when the
  // scale is 0 (where -inf * 0 would be NaN).
  auto probs = [&](const f32x16 (&sc)[2], float bias, i32x8& pf, auto masked) __attribute__((always_inline)) {
    constexpr bool M = decltype(masked)::value;
    float rs = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float e[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float x = sc[w >> 2][4 * (w & 3) + t];
        float arg = fmaf(x, sl2, -bias);
        if (M && x == kNegInf) arg = kNegInf;
        e[t] = fast_exp2(arg);
      }
      rs += (e[0] + e[1]) + (e[2] + e[3]);
      pf[w] = pack_fp8x4(e[0], e[1], e[2], e[3]);
    }
    return rs;
  };
  auto pv_mfmas = [&](const i32x8& pf, const lds8_t* Vc, int hk) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < G::NB; ++n) acc[n] = mfma8(vfrag(Vc, hk, n), pf, acc[n]);
  };

  auto tile = [&](const lds8_t* Kc, const lds8_t* Vc, int key0, auto masked, auto mode) __attribute__((always_inline)) {
    constexpr bool M = decltype(masked)::value;
    constexpr int MODE = decltype(mode)::value;
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      f32x16 s[2];
      // Scores of keys 64 hk .. 64 hk + 63: two 16-byte K reads per MFMA, kAhead8 MFMAs ahead.
      __builtin_amdgcn_sched_barrier(0);
      score_mfmas(s, Kc, hk);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead8, 2 * kAhead8, 0);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma8, 1, 0);
        if (i + kAhead8 < NS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead8, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (M) {
        // Element r of block bl is key key0 + 4 hh + c with the constant c below; it is masked
        // when c exceeds one per-lane threshold (past the length, or after the query row).
        const int base = key0 + 4 * hh;
        const int thr = CAUSAL ? min(L - 1, qrow) - base : L - 1 - base;
#pragma unroll
        for (int bl = 0; bl < 2; ++bl)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 64 * hk + 32 * bl + 8 * (r >> 2) + (r & 3);
            if (c > thr) s[bl][r] = kNegInf;
          }
      }
      float bias;
      if constexpr (MODE == FAST) {
        bias = m_run - (float)kPScaleLog2;  // fixed and finite: p times 64
      } else {
        // Online softmax over this block: the reference moves (and output and sum are
        // rescaled) only for rows whose maximum outgrew it by more than 2^kLagLog2.
        float mx = s[0][0];
#pragma unroll
        for (int bl = 0; bl < 2; ++bl)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[bl][r]);
        mx = max_xor32(mx);
        const float mt = (mx == kNegInf) ? kNegInf : mx * sl2;
        if constexpr (MODE == FIRST) m_seen = fmaxf(m_seen, mt);
        const bool grow = mt > m_run + kLagLog2;  // -inf + 2 = -inf: the first key always moves it
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float m_new = grow ? mt : m_run;
          const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;  // 0 before any visible key
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int n = 0; n < G::NB; ++n) acc[n] *= alpha;
        }
        bias = (m_run == kNegInf ? 0.f : m_run) - (float)kPScaleLog2;  // p times 64
      }
      i32x8 pf;
      l_run += probs(s, bias, pf, masked);
      // P V: per output block four transposing V reads (keys 64 hk + 16 q ..) and one MFMA.
      __builtin_amdgcn_sched_barrier(0);
      pv_mfmas(pf, Vc, hk);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead8, 4 * kAheadV8, 0);
#pragma unroll
      for (int i = 0; i < G::NB; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma8, 1, 0);
        if (i + kAheadV8 < G::NB) __builtin_amdgcn_sched_group_barrier(kSchedDsRead8, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // The LDS loads that follow (the next block's K fragments) may be given the registers
      // that held P and V^T for the MFMAs just issued.  The compiler orders a later write of an
      // MFMA's C operand after the MFMA, but not a later load into its A or B operands, and the
      // 64-deep FP8 MFMA can still be reading those (measured: corrupted accumulators when the
      // loads follow directly).  A vector read of the last MFMA's result is a read-after-write
      // on an MFMA result, which the compiler does order: it waits until that MFMA has written
      // its result, hence read its operands, and MFMAs of one wave complete in issue order.
      // Adding +0 changes nothing but the sign of a zero.
      acc[G::NB - 1][15] += 0.f;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // FAST tiles that need no mask: the two 64-key blocks overlap inside the wave.  Block 1's
  // score products run under block 0's softmax and block 0's P V products under block 1's, so
  // the matrix cores and the vector unit of the wave's SIMD both have work from this wave most
  // of the time (otherwise each block is products, softmax, products in sequence, and only the
  // other wave of the SIMD can fill the gaps).  Between the regions a vector read of the last
  // product issued (x += 0) waits until it has read its operands before the next region's LDS
  // loads may reuse their registers (the FP8 MFMA operand hazard described in tile above).
  auto tile_fast = [&](const lds8_t* Kc, const lds8_t* Vc) __attribute__((always_inline)) {
    constexpr int kValuPerMfma = (120 + NS - 1) / NS;  // a block's softmax over its MFMAs
    const float bias = m_run - (float)kPScaleLog2;    // fixed and finite: p times 64
    f32x16 s0[2], s1[2];
    i32x8 pf0, pf1;
    // S(0): the score products of keys 0..63 (K reads kAhead8 MFMAs ahead).
    __builtin_amdgcn_sched_barrier(0);
    score_mfmas(s0, Kc, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead8, 2 * kAhead8, 0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma8, 1, 0);
      if (i + kAhead8 < NS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead8, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    s0[1][15] += 0.f;
    __builtin_amdgcn_sched_barrier(0);
    // A: S(1) under the softmax of block 0.
    score_mfmas(s1, Kc, 1);
    float rs0 = probs(s0, bias, pf0, std::false_type{});
    // The sums feed l only at the tile's end; without this use the adds (and the exponentials
    // they read) would be moved there, after every product of the tile.
    asm volatile("" : "+v"(rs0));
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead8, 2 * kAhead8, 0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma8, 1, 0);
      if (i + kAhead8 < NS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead8, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu8, kValuPerMfma, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    s1[1][15] += 0.f;
    __builtin_amdgcn_sched_barrier(0);
    // B: P V of block 0 under the softmax of block 1.
    pv_mfmas(pf0, Vc, 0);
    float rs1 = probs(s1, bias, pf1, std::false_type{});
    asm volatile("" : "+v"(rs1));
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead8, 4 * kAheadV8, 0);
#pragma unroll
    for (int i = 0; i < G::NB; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma8, 1, 0);
      if (i + kAheadV8 < G::NB) __builtin_amdgcn_sched_group_barrier(kSchedDsRead8, 4, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu8, (120 + G::NB - 1) / G::NB, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    acc[G::NB - 1][15] += 0.f;
    __builtin_amdgcn_sched_barrier(0);
    // C: P V of block 1.
    pv_mfmas(pf1, Vc, 1);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead8, 4 * kAheadV8, 0);
#pragma unroll
    for (int i = 0; i < G::NB; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma8, 1, 0);
      if (i + kAheadV8 < G::NB) __builtin_amdgcn_sched_group_barrier(kSchedDsRead8, 4, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    acc[G::NB - 1][15] += 0.f;
    __builtin_amdgcn_sched_barrier(0);
    l_run += rs0 + rs1;
  };

  const int n_main = CAUSAL ? min(q0, L) / kBN8 : L / kBN8;
  auto iter = [&](int j, auto parity, auto masked, auto mode) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(parity)::value;
    lds8_t* const Kc = ODD ? K1 : K0;
    lds8_t* const Vc = ODD ? V1 : V0;
    lds8_t* const Kn = ODD ? K0 : K1;
    lds8_t* const Vn = ODD ? V0 : V1;
    if (j + 1 < n_kt) {
      load_tile8<D, NW>(Kn, Kg, (j + 1) * kBN8, L, koff, wave);
      load_tile8<D, NW>(Vn, Vg, (j + 1) * kBN8, L, voff, wave);
    }
    if (j < n_kw) {
      if constexpr (decltype(mode)::value == FAST && !decltype(masked)::value) tile_fast(Kc, Vc);
      else tile(Kc, Vc, j * kBN8, masked, mode);
    }
    wait_loads8();
    __syncthreads();
  };
  using even = std::false_type;
  using odd = std::true_type;
  using unmasked = std::false_type;
  using masked = std::true_type;
  auto run = [&](auto mode) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode)::value;
    using first_mode = std::integral_constant<int, MODE == SAFE ? SAFE : FIRST>;
    // Tile 0 (K_0 and V_0 are loading or loaded): the FAST pass takes its references from it.
    wait_loads8();
    __syncthreads();
    if (0 < n_main) iter(0, even{}, unmasked{}, first_mode{});
    else iter(0, even{}, masked{}, first_mode{});
    if constexpr (MODE == FAST) {
      // Fix the reference: O and l move from the lagging reference to it (a row that saw no
      // key has O = l = 0; it is padding and takes any finite reference).
      const float m_fix = (m_seen == kNegInf ? 0.f : m_seen) + kHeadLog2;
      const float alpha = fast_exp2(m_run - m_fix);
      m_run = m_fix;
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < G::NB; ++n) acc[n] *= alpha;
    }
    int j = 1;
    for (; j + 1 < n_main; j += 2) {
      iter(j, odd{}, unmasked{}, mode);
      iter(j + 1, even{}, unmasked{}, mode);
    }
    if (j < n_main) {
      iter(j, odd{}, unmasked{}, mode);
      ++j;
    }
    for (; j < n_kt; ++j) {
      if (j & 1) iter(j, odd{}, masked{}, mode);
      else iter(j, even{}, masked{}, mode);
    }
  };
  run(std::integral_constant<int, FAST>{});
  // A NaN accumulator: some probability overflowed the fixed reference (or an input is NaN).
  if (__syncthreads_or(acc[0][0] != acc[0][0])) {
#pragma unroll
    for (int n = 0; n < G::NB; ++n) acc[n] = f32x16{};
    m_run = kNegInf;
    l_run = 0.f;
    load_tile8<D, NW>(K0, Kg, 0, L, koff, wave);
    load_tile8<D, NW>(V0, Vg, 0, L, voff, wave);
    run(std::integral_constant<int, SAFE>{});
  }

  // Epilogue: O = v_scale * acc / l (both carry the factor 64); LSE = ln 2 (m + log2 l - 6).
  const float lt = add_xor32(l_run);
  if (qrow < N) {
    const bool valid = qrow < L;
    const float f = valid ? p.v_scale / lt : 0.f;
#pragma unroll
    for (int n = 0; n < G::NB; ++n) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[n][4 * r4 + 0] * f, acc[n][4 * r4 + 1] * f);
        w[1] = pack_bf16x2(acc[n][4 * r4 + 2] * f, acc[n][4 * r4 + 3] * f);
        *reinterpret_cast<u32x2*>(Og + (size_t)qrow * D + n * 32 + 8 * r4 + 4 * hh) = w;
      }
    }
    if (hh == 0) LSEg[qrow] = valid ? (m_run + __log2f(lt) - (float)kPScaleLog2) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL>
hipError_t launch8(const Fp8FwdArgs& a, hipStream_t stream) {
  Params8 p;
  p.q = static_cast<const uint8_t*>(a.q);
  p.k = static_cast<const uint8_t*>(a.k);
  p.v = static_cast<const uint8_t*>(a.v);
  p.o = static_cast<bf16*>(a.o);
  p.lse = a.lse;
  p.seq_lens = a.seq_lens;
  p.H = a.H;
  p.group = a.H / a.Hkv;
  p.Hkv = a.Hkv;
  p.N = a.N;
  p.sl2 = a.scale * a.q_scale * a.k_scale * kLog2e;
  p.v_scale = a.v_scale;
  const long long wide = (long long)a.B * a.H * ((a.N + 8 * kWQ8 - 1) / (8 * kWQ8));
  if (wide >= kCUs8) {
    p.n_qt = (a.N + 8 * kWQ8 - 1) / (8 * kWQ8);
    p.total = a.B * a.H * p.n_qt;
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, 8>), dim3(p.total), dim3(64 * 8), 0, stream, p);
  } else {
    p.n_qt = (a.N + 4 * kWQ8 - 1) / (4 * kWQ8);
    p.total = a.B * a.H * p.n_qt;
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, 4>), dim3(p.total), dim3(64 * 4), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch8<128, true>(a, stream) : launch8<128, false>(a, stream);
  return a.causal ? launch8<64, true>(a, stream) : launch8<64, false>(a, stream);
}

}  // namespace fa
