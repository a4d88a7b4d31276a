// fa_fwd_bf16.hip -- fused attention forward, bf16 storage, fp32 accumulation, gfx950 MFMA.
//
// One workgroup owns BM query rows of one (batch, head) and streams that head's K/V in tiles
// of BN keys through LDS (the fused, tiled scheme of "Gemini 3 Flash的注意力内核重写" -- kernel
// fusion, tiling -- and "FlashAttention优化" §3.1: the query block stays resident and every
// K/V block streams past it).  Per tile it computes scores on the matrix cores, updates the
// running row maximum and row sum with the online-softmax recurrence of "FlashAttention优化"
// §3.2.1, and adds P V on the matrix cores.  Scores and probabilities live only in registers.
// The output is divided by the row sum once at the end (the deferred rescale the "GPU优化" tag
// page attributes to FlashAttention V2) and the natural-log LSE of each row is written beside
// it.
//
// CDNA4 mapping (the pages' A100/H100 tile sizes are prior art, not used):
//  * A wave owns 32 query rows; BN = 64 keys per tile.  A workgroup is 8 waves (256 rows, one
//    workgroup per CU, two waves per SIMD) when that still gives every CU a workgroup.  Smaller
//    grids take 128-row workgroups: with at most one per CU, 8 waves in two key groups (each
//    group streams every other K/V tile; the partial results are combined at the end), else 4
//    waves, two workgroups per CU.  A wave holds its Q^T fragments, one 64 x 32 score tile and
//    the 32 x d output accumulator in registers (<= 256 per lane).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K rows are
//    the A operand (read from LDS), Q^T the B operand (registers).  The accumulator holds one
//    query per lane and 16 keys per lane, so row reductions are in-lane plus one exchange with
//    lane ^ 32 (v_permlane32_swap).  Packed to bf16, a lane's probabilities are already the B
//    operand of O^T += V^T P^T (keys in k-slots), so P never leaves registers.
//  * K and V go from global memory straight into LDS (buffer_load ... lds, no staging
//    registers), into two buffers each; tile j+1 loads while tile j is computed, one barrier per
//    tile.  The 16-byte chunks of a row are XOR-swizzled by row so that the fragment reads are
//    free of bank conflicts.  V stays [key][dim] in LDS; its V^T fragments are read with
//    ds_read_b64_tr_b16, the gfx950 transposing LDS read (each 16-lane group turns a 4-key x
//    16-dim block into 4 consecutive keys per lane).
//  * Inside a tile the score MFMAs run with their fragment reads a few MFMAs ahead; the P V
//    MFMAs run chunk by chunk (16 keys) with the next chunk's probabilities computed under them.
//    A wave raises its issue priority while it issues MFMAs, so the matrix cores of a SIMD
//    switch to the other wave only when this one waits.
//  * The reference maximum of each row is fixed at its first tile (FAST pass) and checked, not
//    tracked: no rescaling in the loop.  A later tile whose probabilities could exceed 2^16
//    raises a flag, and the workgroup then recomputes with the running maximum and rescaling
//    (SAFE pass).  Both give the exact softmax (details at the K/V loop below).
//  * The grid is one workgroup per (batch, head, query tile), remapped so that the tiles of one
//    (batch, kv head) run on the same XCD and share its L2, and so that every XCD gets the same
//    mix of sequences.  Under causal masking the heaviest query tiles are issued first, tiles
//    past the diagonal are never loaded, and a wave whose rows all lie above a tile skips it.
#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tiles.h"
#include "fa_softmax.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kCUs = 256;              // compute units of an MI355X
constexpr int kXcds = 8;               // accelerator complex dies (each with its own L2)

struct Params {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  const int32_t* seq_lens;  // valid rows per sequence, or nullptr
  int H, group, Hkv, N, n_qt, total;
  float sl2;  // scale * log2(e): scores go to the exponent base 2
};

// With per-sequence lengths (varlen prefill): the sequence a workgroup serves, taken in order of
// decreasing length L (ties by index), which is also the order of total work, so the sequences
// holding the heaviest workgroups start first and the light ones fill in behind them.  Every workgroup ranks the sequences itself, one thread per sequence
// against lengths staged in LDS; with more than kMaxRanked sequences the natural order is kept.
// The order changes no result.
constexpr int kMaxRanked = 512;
template <int NW>
__device__ int by_work(const Params& p, int S, int pos, int* buf) {  // S: sequences in the grid
  if (S > kMaxRanked) return pos;
  int* w = buf;                   // key length of each sequence
  int* order = buf + kMaxRanked;  // sequence at each rank
  for (int i = threadIdx.x; i < S; i += 64 * NW)
    w[i] = min(max(p.seq_lens[i], 0), p.N);
  __syncthreads();
  for (int i = threadIdx.x; i < S; i += 64 * NW) {
    int r = 0;
    for (int t = 0; t < S; ++t) r += (w[t] > w[i]) || (w[t] == w[i] && t < i);
    order[r] = i;
  }
  __syncthreads();
  return order[pos];
}

// NG = 1: the NW waves own NW * 32 query rows and share every K/V tile.  NG = 2 (grids too
// small to give each SIMD two waves otherwise): the waves form two groups of NW / 2 over the
// same NW / 2 * 32 rows; group g takes the key tiles t with t % 2 == g, with its own LDS
// buffers, and the two partial results (output, reference maximum, row sum) are combined
// exactly at the end, as the online softmax combines any two blocks of keys
// ("FlashAttention优化" §3.2.2).
// PAIR (causal grids that one round of 256-row tiles would leave to their heaviest tile): the
// workgroup computes query tile i and then tile n_qt - 1 - i, so every workgroup has the same
// number of key tiles to visit.
template <int D, bool CAUSAL, int NW, int NG = 1, bool PAIR = false>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(Params p) {
  static_assert(NG == 1 || NG == 2, "one or two key groups");
  using G = Geo<D>;
  constexpr int NWG = NW / NG;          // waves per key group
  constexpr int kBM = NWG * kWQ;        // query rows per workgroup
  constexpr int kThreads = 64 * NW;
  constexpr int NI_W = LoadGeo<D, NWG>::NI_W;
  // K_0, K_1, V_0, V_1: one tile per key group each (group g's at offset g * TILE).  Separate
  // arrays, so that the compiler sees that reads of one buffer never wait for loads into another.
  __shared__ __attribute__((aligned(1024))) char k0s[NG * G::TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[NG * G::TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[NG * G::TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[NG * G::TILE];
  lds_t* const K0 = (lds_t*)k0s;
  lds_t* const K1 = (lds_t*)k1s;
  lds_t* const V0 = (lds_t*)v0s;
  lds_t* const V1 = (lds_t*)v1s;
  __shared__ int rank_buf[2 * kMaxRanked];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: kept in a scalar register
  const int c32 = lane & 31, hh = lane >> 5;
  const int grp = NG > 1 ? __builtin_amdgcn_readfirstlane(wave / NWG) : 0;  // key group
  const int wq = wave - grp * NWG;  // rows wq * 32 .. +31 of the workgroup's query tile
  const int gofs = grp * G::TILE;   // the group's tile inside each buffer

  // Work unit = (batch, kv head): the group's query heads and their query tiles, which all read
  // the same K/V.  Each XCD runs a contiguous range of logical tiles (shared L2); when the units
  // divide evenly, XCD x takes units x, x+8, x+16, ... so every XCD holds the same mix of
  // sequences (causal work grows with the square of a sequence's length).
  const int lam = xcd_remap(blockIdx.x, p.total);
  const int n_slots = PAIR ? (p.n_qt + 1) / 2 : p.n_qt;  // query tiles (pairs) per head
  const int per_unit = p.group * n_slots;
  const int units = p.total / per_unit;
  int unit = lam / per_unit;
  const int rem = lam - unit * per_unit;
  if (units % kXcds == 0) unit = (unit % (units / kXcds)) * kXcds + unit / (units / kXcds);
  int b = unit / p.Hkv;
  const int g = unit - b * p.Hkv;
  if (p.seq_lens != nullptr) b = by_work<NW>(p, units / p.Hkv, b, rank_buf);  // heaviest first
  // Inside a unit the group's query heads take consecutive slots for each query tile: heads that
  // read the same K/V rows run side by side (shared L2 lines), and every head's heaviest tiles
  // come before any head's lighter ones.
  int qt = rem / p.group;
  const int hi = rem - qt * p.group;
  if (CAUSAL && !PAIR) qt = p.n_qt - 1 - qt;  // heaviest query tiles first
  const int H = p.H, N = p.N;
  const int h = g * p.group + hi;
  const int bh = b * H + h;
  // L: valid rows of this sequence (queries and keys alike).
  int L = N;
  if (p.seq_lens != nullptr) L = min(max(p.seq_lens[b], 0), N);

  const bf16* Qg = p.q + (size_t)bh * N * D;
  const bf16* Kg = p.k + (size_t)(b * p.Hkv + g) * N * D;
  const bf16* Vg = p.v + (size_t)(b * p.Hkv + g) * N * D;
  bf16* Og = p.o + (size_t)bh * N * D;
  float* LSEg = p.lse + (size_t)bh * N;

  // One query tile: the whole computation of its rows (returns early for a tile of padding rows
  // and, with two key groups, for group 1 once it has handed over its partial result).
  auto work = [&](const int qt) __attribute__((always_inline)) {
    const int q0 = qt * kBM;
    if (q0 >= L) {  // every row of this tile is padding: O = 0, LSE = -inf
      const int rows = min(kBM, N - q0);
      const u32x4 zero = {0u, 0u, 0u, 0u};
      for (int i = tid; i < rows * G::CPR; i += kThreads)
        *reinterpret_cast<u32x4*>(Og + (size_t)q0 * D + i * 8) = zero;
      for (int r = tid; r < rows; r += kThreads) LSEg[q0 + r] = kNegInf;
      return;
    }

    const int kv_end = CAUSAL ? min(L, q0 + kBM) : L;   // keys this workgroup needs
    const int n_kt = (kv_end + kBN - 1) / kBN;
    const int qw0 = q0 + wq * kWQ;
    const int qrow = qw0 + c32;
    // Tiles this wave needs (fewer than n_kt on the causal diagonal).
    const int n_kw = CAUSAL ? min(n_kt, (min(L, qw0 + kWQ) + kBN - 1) / kBN) : n_kt;
    const float sl2 = p.sl2;
    int koff[NI_W], voff[NI_W];
    tile_offsets<D, NWG, false>(koff, wq, lane);
    tile_offsets<D, NWG, true>(voff, wq, lane);
    auto load_kv = [&](lds_t* Kd, lds_t* Vd, int jt) __attribute__((always_inline)) {
      load_tile<D, NWG>(Kd + gofs, Kg, jt * kBN, L, koff, wq);
      load_tile<D, NWG>(Vd + gofs, Vg, jt * kBN, L, voff, wq);
    };

    // Issue the first loads before anything else: K_0 and V_0.
    if (NG == 1 || grp < n_kt) load_kv(K0, V0, grp);  // the group's first tile

    // Q^T fragments (B operand of S^T = K Q^T), resident for the whole kernel; zero for padding
    // rows, so that whatever they hold (NaN included) cannot reach their zero output.
    bf16x8 qf[G::KC];
#pragma unroll
    for (int c = 0; c < G::KC; ++c) {
      qf[c] = qrow < L ? *reinterpret_cast<const bf16x8*>(Qg + (size_t)qrow * D + c * 16 + hh * 8)
                        : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    FragAddr<D> fa = frag_addr<D>(lane);
    if constexpr (NG > 1) {
#pragma unroll
      for (int c = 0; c < G::KC; ++c) fa.k[c] += gofs;
#pragma unroll
      for (int n = 0; n < G::NB; ++n) fa.v[n] += gofs;
    }

    f32x16 acc[G::NB];
#pragma unroll
    for (int n = 0; n < G::NB; ++n) acc[n] = f32x16{};
    float m_run = kNegInf;  // reference maximum (log2 units); -inf until a key is seen
    float l_run = 0.f;      // this lane's share of the row sum (relative to m_run)

    f32x16 sA[2];

    // The K/V loop runs in one of two modes.
    //  * FAST (first try): every row keeps the maximum of its first tile as a fixed reference, so
    //    nothing accumulated is ever rescaled and later tiles need no maximum at all.  A tile in
    //    which some lane's share of the row sum exceeds 2^kTau -- the only way one of its
    //    probabilities can exceed 2^kTau -- raises a flag; otherwise every probability stays far
    //    inside the bf16/fp32 range.
    //  * SAFE: the running maximum with a rescale of O and l whenever it grows
    //    ("FlashAttention优化" §3.2.1), taken only if some wave of the workgroup raised the flag.
    // With a fixed reference the output and the row sum are the same sums the recurrence forms, so
    // both modes give the exact softmax.
    enum { FIRST = 0, FAST = 1, SAFE = 2 };
    bool flagged = false;
    auto tile = [&](const lds_t* Kc, const lds_t* Vc, int key0, auto masked,
                    auto mode) __attribute__((always_inline)) {
      constexpr bool M = decltype(masked)::value;
      constexpr int MODE = decltype(mode)::value;
      scores<D>(sA, Kc, fa, qf);
      if constexpr (M) mask_scores<CAUSAL>(sA, key0, L, qrow, hh);
      if constexpr (MODE == FAST) {
        // No tile maximum: every probability is at most the lane's share of the tile's row sum,
        // so that sum exceeding 2^kTau is the test that some score outgrew the reference.
        const float rs = softmax_pv<D, M, false>(acc, Vc, fa, sA, sl2, m_run, 1.f);
        flagged |= rs > kMaxProb;
        l_run += rs;
        return;
      }
      const float mx = tile_max(sA);
      const float mt = (mx == kNegInf) ? kNegInf : mx * sl2;
      if constexpr (MODE == SAFE) {
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;   // -inf only before any visible key
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        l_run = fmaf(alpha, l_run, softmax_pv<D, M, true>(acc, Vc, fa, sA, sl2, m_use, alpha));
      } else {
        m_run = (mt == kNegInf) ? 0.f : mt;
        l_run += softmax_pv<D, M, false>(acc, Vc, fa, sA, sl2, m_run, 1.f);
      }
    };

    // Iteration j computes the group's tile j * NG + grp from buffers j % 2 while its next tile
    // loads into the others.  The buffer is fixed per instantiation, so every LDS access refers to
    // one known buffer and the compiler never waits for the loads in flight.  Tiles [0, n_main)
    // need no mask for any wave of the workgroup; the remaining ones (the causal diagonal, the
    // ragged end) are masked.  Iterations are counted for the whole workgroup (n_it, one barrier
    // each) and per wave (n_iw, the iterations whose tile the wave needs).
    const int n_main = CAUSAL ? min(q0, L) / kBN : L / kBN;
    const int n_mi = n_main / NG;                  // iterations whose tiles all need no mask
    const int n_it = (n_kt + NG - 1) / NG;
    const int n_iw = (n_kw - grp + NG - 1) / NG;
    auto iter = [&](int j, auto parity, auto masked, auto mode) __attribute__((always_inline)) {
      constexpr bool ODD = decltype(parity)::value;
      lds_t* const Kc = ODD ? K1 : K0;
      lds_t* const Vc = ODD ? V1 : V0;
      lds_t* const Kn = ODD ? K0 : K1;
      lds_t* const Vn = ODD ? V0 : V1;
      if ((j + 1) * NG + grp < n_kt) load_kv(Kn, Vn, (j + 1) * NG + grp);
      if (j < n_iw) tile(Kc, Vc, (j * NG + grp) * kBN, masked, mode);
      wait_loads();
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
      wait_loads();
      __syncthreads();
      if (0 < n_mi) iter(0, even{}, unmasked{}, first_mode{});
      else iter(0, even{}, masked{}, first_mode{});
      int j = 1;
      for (; j + 1 < n_mi; j += 2) {
        iter(j, odd{}, unmasked{}, mode);
        iter(j + 1, even{}, unmasked{}, mode);
      }
      if (j < n_mi) {
        iter(j, odd{}, unmasked{}, mode);
        ++j;
      }
      for (; j < n_it; ++j) {
        if (j & 1) iter(j, odd{}, masked{}, mode);
        else iter(j, even{}, masked{}, mode);
      }
    };
    run(std::integral_constant<int, FAST>{});
    if (__syncthreads_or(flagged)) {  // some row's maximum outgrew its reference: exact fallback
#pragma unroll
      for (int n = 0; n < G::NB; ++n) acc[n] = f32x16{};
      m_run = kNegInf;
      l_run = 0.f;
      if (NG == 1 || grp < n_kt) load_kv(K0, V0, grp);
      run(std::integral_constant<int, SAFE>{});
    }

    float lt = add_xor32(l_run);
    if constexpr (NG > 1) {
      // Combine the two key groups' partial results for the same rows: group 1 hands its output
      // accumulator, reference maximum and row sum over LDS (the tile buffers, free now) to the
      // wave of group 0 that owns the same rows, lane for lane (the accumulator layouts match).
      // A group whose row sum is 0 saw no key of the row and drops out; group 0 always holds the
      // row's first key.
      constexpr int kAccB = 64 * G::NB * 16 * 4;  // accumulator bytes per wave
      static_assert(NWG == 4 && 2 * kAccB == NG * G::TILE, "two waves' accumulators per buffer");
      f32x4* const xa = reinterpret_cast<f32x4*>((wq < 2 ? k0s : k1s) + (wq & 1) * kAccB);
      float* const xm = reinterpret_cast<float*>(v0s) + wq * 128;
      __syncthreads();  // every wave is done with the tile buffers
      if (grp == 1) {
#pragma unroll
        for (int n = 0; n < G::NB; ++n)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 v = {acc[n][4 * r4], acc[n][4 * r4 + 1], acc[n][4 * r4 + 2],
                             acc[n][4 * r4 + 3]};
            xa[(n * 4 + r4) * 64 + lane] = v;
          }
        xm[lane] = m_run;
        xm[64 + lane] = lt;
      }
      __syncthreads();
      if (grp == 1) return;
      const float m1 = xm[lane], lt1 = xm[64 + lane];
      const float m0 = lt > 0.f ? m_run : kNegInf;
      const float mm = fmaxf(m0, lt1 > 0.f ? m1 : kNegInf);
      const float a0 = lt > 0.f ? fast_exp2(m_run - mm) : 0.f;
      const float a1 = lt1 > 0.f ? fast_exp2(m1 - mm) : 0.f;
#pragma unroll
      for (int n = 0; n < G::NB; ++n)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 v = xa[(n * 4 + r4) * 64 + lane];
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[n][4 * r4 + t] = acc[n][4 * r4 + t] * a0 + v[t] * a1;
        }
      lt = lt * a0 + lt1 * a1;
      m_run = mm;
    }

    // Epilogue: O = acc / l once; LSE = ln 2 * (m + log2 l).
    if (qrow < N) {
      const bool valid = qrow < L;
      const float inv = valid ? 1.f / lt : 0.f;
#pragma unroll
      for (int n = 0; n < G::NB; ++n) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          u32x2 w;
          w[0] = pack_bf16x2(acc[n][4 * r4 + 0] * inv, acc[n][4 * r4 + 1] * inv);
          w[1] = pack_bf16x2(acc[n][4 * r4 + 2] * inv, acc[n][4 * r4 + 3] * inv);
          *reinterpret_cast<u32x2*>(Og + (size_t)qrow * D + n * 32 + 8 * r4 + 4 * hh) = w;
        }
      }
      if (hh == 0) LSEg[qrow] = valid ? (m_run + __log2f(lt)) * kLn2 : kNegInf;
    }
  };
  work(qt);
  if constexpr (PAIR) {
    const int qt2 = p.n_qt - 1 - qt;
    if (qt2 != qt) {
      __syncthreads();  // group 0 has read group 1's partial result out of the tile buffers
      work(qt2);
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  Params p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.o = static_cast<bf16*>(a.o);
  p.lse = a.lse;
  p.seq_lens = a.seq_lens;
  p.H = a.H;
  p.group = a.H / a.Hkv;
  p.Hkv = a.Hkv;
  p.N = a.N;
  p.sl2 = a.scale * kLog2e;
  // Eight waves (256 rows) per workgroup share each K/V tile in LDS when that still gives every
  // CU a workgroup.  Otherwise 128-row workgroups: eight waves in two key groups when there are
  // at most as many workgroups as CUs (two waves per SIMD where four waves would leave one),
  // else four waves, two workgroups per CU.
  const long long wide = (long long)a.B * a.H * ((a.N + 8 * kWQ - 1) / (8 * kWQ));
  const long long pairs = (long long)a.B * a.H * (((a.N + 4 * kWQ - 1) / (4 * kWQ) + 1) / 2);
  if constexpr (CAUSAL) {
    if (wide >= kCUs && wide < 2 * kCUs && pairs >= kCUs) {
      // One or two rounds of 256-row causal tiles run at the pace of the heaviest: 128-row
      // tiles in pairs (i, n - 1 - i) instead, two key groups of four waves each.
      p.n_qt = (a.N + 4 * kWQ - 1) / (4 * kWQ);
      p.total = (int)pairs;
      hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 8, 2, true>), dim3(p.total), dim3(64 * 8), 0,
                         stream, p);
      return hipGetLastError();
    }
  }
  if (wide >= kCUs) {
    p.n_qt = (a.N + 8 * kWQ - 1) / (8 * kWQ);
    p.total = a.B * a.H * p.n_qt;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 8>), dim3(p.total), dim3(64 * 8), 0, stream, p);
  } else {
    p.n_qt = (a.N + 4 * kWQ - 1) / (4 * kWQ);
    p.total = a.B * a.H * p.n_qt;
    if (p.total <= kCUs)
      hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 8, 2>), dim3(p.total), dim3(64 * 8), 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 4>), dim3(p.total), dim3(64 * 4), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
