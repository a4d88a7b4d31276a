// fa_prefill_paged.hip -- chunked prefill against a paged KV cache, gfx950.
//
// Each sequence's newest Q_b tokens attend, causally with the offset L_b - Q_b, to the L_b
// tokens of the sequence held in the cache in fixed-size blocks that a block table addresses
// (the paged cache of ocdem's "非连续块Gather" §二.1; the chunked prefill of ijyty §3.2).  The
// arithmetic is the fused forward's: scores and probabilities stay in registers, K/V tiles of 64
// keys stream through LDS, the online softmax of "FlashAttention优化" §3.2.1 with a fixed
// per-row reference (and an exact fallback with the running maximum).
//
// What differs from the contiguous forward is the shape of the work: chunk lengths and context
// lengths vary per sequence and are known only on the device.  Three kernels:
//  * plan (one workgroup): reads the lengths and writes the work items into the caller's
//    workspace (the plan's rules are in fa_prefill_plan.h): the query heads that share a kv head
//    go into one item, 32 rows each, so a short chunk still fills the four waves; long key loops
//    are split into pieces of at most T tiles ("Split-KV"), T set from the total work so that no
//    item is longer than twice a workgroup's average share; items are placed so that each XCD
//    runs the items of the same kv heads side by side, heaviest first.
//  * attend: one workgroup per item (two per CU).  An unsplit item writes O and the LSE; a piece
//    writes its unnormalised output, reference maximum and row sum to a partials slot.  The
//    hardware dispatcher gives each freed slot the next item, so no counter is shared.
//  * merge: the pieces of each split block combined exactly -- M = max m_s,
//    O = sum 2^(m_s - M) O_s / sum 2^(m_s - M) l_s, LSE = ln 2 (M + log2 sum 2^(m_s - M) l_s)
//    ("FlashAttention优化" §3.2.2).
// Stream order carries the dependencies: the plan's writes are complete when attend starts,
// attend's partials when merge starts.
#include "fa_device.h"
#include "fa_launch.h"
#include "fa_prefill_plan.h"
#include "fa_softmax.h"
#include "fa_tiles.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPageRows = plan::kPageRows;

struct PrefillParams {
  const bf16* q;   // [S, Hq, max_q, d]
  const bf16* k;   // key cache [num_blocks, 16, Hkv, d]
  const bf16* v;   // value cache
  bf16* o;         // [S, Hq, max_q, d]
  float* lse;      // [S, Hq, max_q]
  const int32_t* seq_lens;
  const int32_t* q_lens;
  const int32_t* table;  // [S, max_blocks]
  plan::Shape shape;
  plan::Bufs w;
  float* opart;    // [slots][128 pairs][d]
  float* mpart;    // [slots][128 pairs]
  float* lpart;
  int Hq, Hkv, group, max_blocks, num_blocks;
  float sl2;       // scale * log2(e)
};

// Per-lane byte offsets of this wave's direct loads when the tile rows come from a paged cache:
// tile row r lives at slot r % 16 of its block, rows of one block are Hkv * d elements apart,
// and the chunk swizzle is the tile's (by tile row).  Each load covers rows of one block.
template <int D, int NW, bool IS_V>
__device__ __forceinline__ void tile_offsets_paged(int* off, int wave, int lane, int row_elems) {
  using G = Geo<D>;
  constexpr int NI_W = LoadGeo<D, NW>::NI_W;
#pragma unroll
  for (int t = 0; t < NI_W; ++t) {
    const int row = (wave * NI_W + t) * G::RPI + lane / G::CPR;
    const int chunk = (lane % G::CPR) ^ (IS_V ? G::swz_v(row) : G::swz_k(row));
    off[t] = (row % kPageRows) * row_elems * 2 + chunk * 16;
  }
}

// Direct global -> LDS copy of this wave's rows of one tile from a paged cache: all of them lie
// in one physical block (bid), whose buffer resource ends at the sequence's last valid token.
template <int D, int NW>
__device__ __forceinline__ void load_tile_paged(lds_t* dst, const bf16* cache, int bid, int g,
                                                int valid_rows, int Hkv, const int* off, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NI_W = LoadGeo<D, NW>::NI_W;
  const int bytes = __builtin_amdgcn_readfirstlane(
      valid_rows > 0 ? ((valid_rows - 1) * Hkv * D + D) * 2 : 0);
  const uintptr_t base = reinterpret_cast<uintptr_t>(
      cache + ((size_t)bid * kPageRows * Hkv + g) * D);
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

// ---------------------------------------------------------------------------------------------
// Plan: one workgroup runs the phases of fa_prefill_plan.h, a barrier between phases.

// Exclusive prefix sum of v[0 .. n) in place by one wave (each lane a contiguous chunk, then a
// scan of the chunk sums across the lanes); returns the total to every lane.
__device__ long long wave_exclusive_scan(int* v, int n, int lane) {
  const int per = (n + 63) / 64;
  const int lo = min(lane * per, n), hi = min(lo + per, n);
  long long sum = 0;
  for (int i = lo; i < hi; ++i) sum += v[i];
  long long inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  long long run = inc - sum;
  for (int i = lo; i < hi; ++i) {
    const int x = v[i];
    v[i] = (int)run;
    run += x;
  }
  return __shfl(inc, 63, 64);
}

// SMALL (S <= kMaxRanked, chosen by the host): the per-sequence arrays live in LDS, and the
// compiler sees that they do, so their reads never wait for the item stores in flight.
template <bool SMALL>
__global__ void __launch_bounds__(kPlanThreads) prefill_plan_kernel(PrefillParams p) {
  const plan::Shape s = p.shape;
  const int tid = threadIdx.x;
  __shared__ int keys[plan::kMaxRanked];
  // Per-sequence arrays in LDS when the sequences are few enough (the common case), else in the
  // workspace.
  __shared__ int seq_s[9 * plan::kMaxRanked];
  __shared__ int pos_s[2 * plan::kXcds * plan::kMaxRanked];
  __shared__ int hdr_s[plan::kHdrInts];  // the header is built here and copied out at the end
  plan::Bufs w = p.w;
  w.hdr = hdr_s;
  if constexpr (SMALL) {
    w.order = seq_s;
    w.n_items = seq_s + plan::kMaxRanked;
    w.n_zero = seq_s + 2 * plan::kMaxRanked;
    w.n_slots = seq_s + 3 * plan::kMaxRanked;
    w.n_entries = seq_s + 4 * plan::kMaxRanked;
    w.slot_base = seq_s + 5 * plan::kMaxRanked;
    w.entry_base = seq_s + 6 * plan::kMaxRanked;
    w.len_k = seq_s + 7 * plan::kMaxRanked;
    w.len_q = seq_s + 8 * plan::kMaxRanked;
    w.pos_real = pos_s;
    w.pos_zero = pos_s + plan::kXcds * plan::kMaxRanked;
  }
  __shared__ long long wsum[kPlanThreads / 64];
  __shared__ long long tot[2 * plan::kXcds + 2];
  __shared__ int T_s;

  // Order: longest key length first.
  if constexpr (SMALL) {
    for (int i = tid; i < s.S; i += kPlanThreads) keys[i] = plan::seq_keys(s, p.seq_lens[i]);
    __syncthreads();
    for (int i = tid; i < s.S; i += kPlanThreads) plan::rank_one(s.S, keys, i, w.order);
  } else {
    for (int i = tid; i < s.S; i += kPlanThreads) w.order[i] = i;
  }
  // Total key tiles W -> split length T.
  long long t = 0;
  for (int i = tid; i < s.S; i += kPlanThreads) {
    const int L = plan::seq_keys(s, p.seq_lens[i]);
    t += plan::seq_tiles(s, L, plan::seq_queries(s, L, p.q_lens[i]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o, 64);
  if ((tid & 63) == 0) wsum[tid >> 6] = t;
  __syncthreads();
  if (tid == 0) {
    long long W = 0;
    for (int i = 0; i < kPlanThreads / 64; ++i) W += wsum[i];
    T_s = plan::split_tiles(W * plan::units_per_seq(s), s.R);
  }
  __syncthreads();
  const int T = T_s;
  for (int r = tid; r < s.S; r += kPlanThreads) plan::count_one(s, p.seq_lens, p.q_lens, T, r, w);
  __syncthreads();
  for (int r = tid; r < s.S; r += kPlanThreads) plan::scan_inputs(s, r, w);
  __syncthreads();
  // 18 prefix sums (real and zero items of each list, slots, merge entries), one wave each.
  for (int a = tid >> 6; a < 2 * plan::kXcds + 2; a += kPlanThreads / 64) {
    int* v = a < plan::kXcds ? w.pos_real + a * s.S
           : a < 2 * plan::kXcds ? w.pos_zero + (a - plan::kXcds) * s.S
           : a == 2 * plan::kXcds ? w.slot_base : w.entry_base;
    const long long total = wave_exclusive_scan(v, s.S, tid & 63);
    if ((tid & 63) == 0) tot[a] = total;
  }
  __syncthreads();
  if (tid == 0) plan::header(s, T, tot, w);
  __syncthreads();
  // Items: one task per (unit, query block); units of sequences with a split block serially.
  const int units = s.S * plan::units_per_seq(s);
  const int tasks = units * plan::blocks_per_unit(s);
  for (int t = tid; t < tasks; t += kPlanThreads) plan::emit_task(s, tot, t, w);
  for (int u = tid; u < units; u += kPlanThreads) plan::emit_split(s, T, u, w);
  for (int i = tid; i < plan::kHdrInts; i += kPlanThreads) p.w.hdr[i] = hdr_s[i];
}

// ---------------------------------------------------------------------------------------------
// Attend: NW waves (4: two workgroups per CU; 8: one, every K/V tile shared by all eight); wave
// w serves query head hw = w % HP of the item's head subset and rows rb * 32 .. rb * 32 + 31
// (rb = w / HP) of its query block.  All waves share every K/V tile.
template <int D, int HP, int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_attend_kernel(PrefillParams p) {
  using G = Geo<D>;
  constexpr int RPH = kWQ * NW / HP;    // query rows per head of an item
  constexpr int NI_W = LoadGeo<D, NW>::NI_W;
  constexpr int kPairs = kWQ * NW;      // (head, row) pairs of an item: one partials slot
  __shared__ __attribute__((aligned(1024))) char k0s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[G::TILE];
  lds_t* const K0 = (lds_t*)k0s;
  lds_t* const K1 = (lds_t*)k1s;
  lds_t* const V0 = (lds_t*)v0s;
  lds_t* const V1 = (lds_t*)v1s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: kept in a scalar register
  const int c32 = lane & 31, hh = lane >> 5;
  const int hw = wave % HP, rb = wave / HP;
  const plan::Shape& s = p.shape;
  const int N = s.max_q;
  const int nu = plan::units_per_seq(s);
  const int n_qb = plan::blocks_per_unit(s);
  const long long max_slots = plan::max_split_slots(s);
  const int* const hdr = p.w.hdr;

  int koff[NI_W], voff[NI_W];
  tile_offsets_paged<D, NW, false>(koff, wave, lane, p.Hkv * D);
  tile_offsets_paged<D, NW, true>(voff, wave, lane, p.Hkv * D);
  const FragAddr<D> fa = frag_addr<D>(lane);
  // This wave's rows of every tile lie in one block, block `wblk` of the tile's kBN / 16.
  const int wblk = __builtin_amdgcn_readfirstlane(wave * NI_W * G::RPI / kPageRows);

  // This workgroup's item: position blockIdx.x of the dense array (read by every lane; the
  // address is uniform).
  const int wpos = blockIdx.x;
  if (wpos >= hdr[plan::kHdrPositions]) return;
  const int* item = p.w.items + (size_t)wpos * plan::kItemInts;
  const int b = __builtin_amdgcn_readfirstlane(item[0]);
  if (b < 0) return;  // an empty position
  const int hg = __builtin_amdgcn_readfirstlane(item[1]);
  const int qb = __builtin_amdgcn_readfirstlane(item[2]);
  const int t0 = __builtin_amdgcn_readfirstlane(item[3]);
  const int t1 = __builtin_amdgcn_readfirstlane(item[4]);
  const int slot = __builtin_amdgcn_readfirstlane(item[5]);
  if (b >= s.S || hg < 0 || hg >= nu || qb < 0 || qb >= n_qb || slot < plan::kZeroItem ||
      slot >= max_slots)
    return;  // never produced by the plan
  const int L = plan::seq_keys(s, p.seq_lens[b]);
  const int Lq = plan::seq_queries(s, L, p.q_lens[b]);
  const int off = L - Lq;
  const int g = hg / s.hgk;
  const int h = g * p.group + (hg - g * s.hgk) * HP + hw;
  const int q0 = qb * RPH;
  const int qw0 = q0 + rb * kWQ;
  const int qrow = qw0 + c32;
  const size_t bh = (size_t)b * p.Hq + h;
  bf16* const Og = p.o + bh * N * D;
  float* const LSEg = p.lse + bh * N;

  if (slot == plan::kZeroItem) {  // rows past the chunk: O = 0, LSE = -inf
    if (qrow < N) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        *reinterpret_cast<u32x4*>(Og + (size_t)qrow * D + c * 16 + hh * 8) = zero;
      if (hh == 0) LSEg[qrow] = kNegInf;
    }
    return;
  }

  const int kv_end = min(L, off + q0 + RPH);              // keys the item's rows may see
  const int n_kt = (kv_end + kBN - 1) / kBN;
  if (t0 < 0 || t1 <= t0 || t1 > n_kt) return;           // never produced by the plan
  const int n_it = t1 - t0;                               // tiles of this item
  // Tiles this wave needs: none if all its rows are padding, fewer on the causal diagonal.
  const int n_kw = qw0 >= Lq ? 0 : min(n_kt, (min(L, off + qw0 + kWQ) + kBN - 1) / kBN);
  const int n_iw = min(max(n_kw - t0, 0), n_it);
  // Tiles before n_main need no mask for any row of the item.
  const int n_main = min(off + q0, L) / kBN;
  const int n_mi = min(max(n_main - t0, 0), n_it);
  const float sl2 = p.sl2;

  // Block ids are read by scalar loads (the table is read-only and the address uniform): a
  // vector load would be waited for through the in-order vector-memory counter, behind the
  // tile loads issued just before it.
  const int* trow = p.table + (size_t)b * p.max_blocks;
  auto block_id = [&](int jt) __attribute__((always_inline)) {
    const int blk = jt * (kBN / kPageRows) + wblk;
    return blk * kPageRows < L ? *(const __attribute__((address_space(4))) int*)(trow + blk) : 0;
  };
  auto load_kv = [&](lds_t* Kd, lds_t* Vd, int jt, int bid) __attribute__((always_inline)) {
    // A block id outside the pool gets an empty resource: its rows read as zeros.
    const bool in_pool = (unsigned)bid < (unsigned)p.num_blocks;
    const int valid = in_pool ? min(max(L - (jt * kBN + wblk * kPageRows), 0), kPageRows) : 0;
    bid = in_pool ? bid : 0;
    load_tile_paged<D, NW>(Kd, p.k, bid, g, valid, p.Hkv, koff, wave);
    load_tile_paged<D, NW>(Vd, p.v, bid, g, valid, p.Hkv, voff, wave);
  };
  int bid_next = 0;
  load_kv(K0, V0, t0, block_id(t0));
  if (1 < n_it) bid_next = block_id(t0 + 1);

  // Q^T fragments of this wave's head and rows; zero for padding rows.
  const bf16* Qg = p.q + bh * N * D;
  bf16x8 qf[G::KC];
#pragma unroll
  for (int c = 0; c < G::KC; ++c) {
    qf[c] = qrow < Lq ? *reinterpret_cast<const bf16x8*>(Qg + (size_t)qrow * D + c * 16 + hh * 8)
                      : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }

  f32x16 acc[G::NB];
#pragma unroll
  for (int n = 0; n < G::NB; ++n) acc[n] = f32x16{};
  float m_run = kNegInf;  // reference maximum (log2 units)
  float l_run = 0.f;      // this lane's share of the row sum (relative to m_run)
  f32x16 sA[2];

  // FAST: the first tile's row maxima are fixed references; a tile whose probabilities could
  // exceed 2^kTau raises a flag.  SAFE (only if some wave raised it): the running maximum with
  // rescaling.  Both give the exact softmax of the item's keys.
  enum { FIRST = 0, FAST = 1, SAFE = 2 };
  bool flagged = false;
  auto tile = [&](const lds_t* Kc, const lds_t* Vc, int key0, auto masked, auto mode) __attribute__((always_inline)) {
    constexpr bool M = decltype(masked)::value;
    constexpr int MODE = decltype(mode)::value;
    scores<D>(sA, Kc, fa, qf);
    if constexpr (M) mask_scores<true>(sA, key0, L, qrow + off, hh);
    if constexpr (MODE == FAST) {
      const float rs = softmax_pv<D, M, false>(acc, Vc, fa, sA, sl2, m_run, 1.f);
      flagged |= rs > kMaxProb;
      l_run += rs;
      return;
    }
    const float mx = tile_max(sA);
    const float mt = (mx == kNegInf) ? kNegInf : mx * sl2;
    if constexpr (MODE == SAFE) {
      const float m_new = fmaxf(m_run, mt);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      l_run = fmaf(alpha, l_run, softmax_pv<D, M, true>(acc, Vc, fa, sA, sl2, m_use, alpha));
    } else {
      m_run = (mt == kNegInf) ? 0.f : mt;
      l_run += softmax_pv<D, M, false>(acc, Vc, fa, sA, sl2, m_run, 1.f);
    }
  };
  // Iteration j computes tile t0 + j from buffers j % 2 while tile t0 + j + 1 loads into the
  // others; one barrier per iteration.
  auto iter = [&](int j, auto parity, auto masked, auto mode) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(parity)::value;
    lds_t* const Kc = ODD ? K1 : K0;
    lds_t* const Vc = ODD ? V1 : V0;
    lds_t* const Kn = ODD ? K0 : K1;
    lds_t* const Vn = ODD ? V0 : V1;
    if (j + 1 < n_it) {
      load_kv(Kn, Vn, t0 + j + 1, bid_next);
      if (j + 2 < n_it) bid_next = block_id(t0 + j + 2);
    }
    if (j < n_iw) tile(Kc, Vc, (t0 + j) * kBN, masked, mode);
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
  if (__syncthreads_or(flagged)) {
#pragma unroll
    for (int n = 0; n < G::NB; ++n) acc[n] = f32x16{};
    m_run = kNegInf;
    l_run = 0.f;
    load_kv(K0, V0, t0, block_id(t0));
    if (1 < n_it) bid_next = block_id(t0 + 1);
    run(std::integral_constant<int, SAFE>{});
  }

  const float lt = add_xor32(l_run);
  if (slot == plan::kDirect) {
    // O = acc / l; LSE = ln 2 * (m + log2 l).
    if (qrow < N) {
      const bool valid = qrow < Lq;
      const float inv = valid ? 1.f / lt : 0.f;
#pragma unroll
      for (int n = 0; n < G::NB; ++n) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          u32x2 wv;
          wv[0] = pack_bf16x2(acc[n][4 * r4 + 0] * inv, acc[n][4 * r4 + 1] * inv);
          wv[1] = pack_bf16x2(acc[n][4 * r4 + 2] * inv, acc[n][4 * r4 + 3] * inv);
          *reinterpret_cast<u32x2*>(Og + (size_t)qrow * D + n * 32 + 8 * r4 + 4 * hh) = wv;
        }
      }
      if (hh == 0) LSEg[qrow] = valid ? (m_run + __log2f(lt)) * kLn2 : kNegInf;
    }
  } else {
    // A piece: its unnormalised output, reference maximum and row sum, (head, row) pair
    // hw * RPH + rb * 32 + c32 of the slot.  A row that saw none of the piece's keys has l = 0.
    const size_t pair = (size_t)slot * kPairs + hw * RPH + rb * kWQ + c32;
    float* const op = p.opart + pair * D;
#pragma unroll
    for (int n = 0; n < G::NB; ++n) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 v4 = {acc[n][4 * r4], acc[n][4 * r4 + 1], acc[n][4 * r4 + 2], acc[n][4 * r4 + 3]};
        *reinterpret_cast<f32x4*>(op + n * 32 + 8 * r4 + 4 * hh) = v4;
      }
    }
    if (hh == 0) {
      p.mpart[pair] = m_run;
      p.lpart[pair] = lt;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Merge: pairs / 64 workgroups per split query block (merge entry), four threads per (head, row)
// pair, each combining D / 4 dimensions.  One pass over the pieces, four at a time with all their
// loads in flight, rescaling the running sums whenever the reference grows (the online merge of
// "FlashAttention优化" §3.2.2): a block costs about np / 4 memory latencies.
constexpr int kMergeTpp = 4;                  // threads per (head, row) pair
constexpr int kMergePairs = 256 / kMergeTpp;  // pairs per workgroup
constexpr int kMergeAhead = 4;                // pieces loaded together
template <int D, int HP>
__global__ void __launch_bounds__(256) prefill_merge_kernel(PrefillParams p) {
  constexpr int DQ = D / kMergeTpp;  // dimensions per thread
  constexpr int NV = DQ / 4;
  const plan::Shape& s = p.shape;
  const int RPH = s.rph;                         // = pairs / HP
  const int wgs = s.pairs / kMergePairs;         // workgroups per merge entry
  const int e = blockIdx.x / wgs;
  const int* hdr = p.w.hdr;
  if (e >= hdr[plan::kHdrMerge]) return;
  const int* ent = p.w.merge + (size_t)e * plan::kMergeInts;
  const int b = ent[0], hg = ent[1], qb = ent[2], slot0 = ent[3], np = ent[4];
  if (b < 0 || b >= s.S || hg < 0 || hg >= plan::units_per_seq(s) || qb < 0 ||
      qb >= plan::blocks_per_unit(s) || np < 2 || slot0 < 0 ||
      (long long)slot0 + np > plan::max_split_slots(s))
    return;  // never produced by the plan
  const int N = s.max_q;
  const int L = plan::seq_keys(s, p.seq_lens[b]);
  const int Lq = plan::seq_queries(s, L, p.q_lens[b]);
  const int g = hg / s.hgk;
  const int pair = (blockIdx.x % wgs) * kMergePairs + threadIdx.x / kMergeTpp;
  const int part = threadIdx.x % kMergeTpp;
  const int hw = pair / RPH;
  const int row = qb * RPH + pair % RPH;
  if (row >= N) return;
  const int h = g * p.group + (hg - g * s.hgk) * HP + hw;
  const size_t bh = (size_t)b * p.Hq + h;
  bf16* const out = p.o + (bh * N + row) * D + part * DQ;
  if (row >= Lq) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < DQ / 8; ++c) reinterpret_cast<u32x4*>(out)[c] = zero;
    if (part == 0) p.lse[bh * N + row] = kNegInf;
    return;
  }
  const size_t at0 = (size_t)slot0 * s.pairs + pair;
  f32x4 num[NV];
#pragma unroll
  for (int c = 0; c < NV; ++c) num[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float M = kNegInf, den = 0.f;
  for (int sp = 0; sp < np; sp += kMergeAhead) {
    float m[kMergeAhead], l[kMergeAhead];
    f32x4 x[kMergeAhead][NV];
#pragma unroll
    for (int u = 0; u < kMergeAhead; ++u) {
      const size_t at = at0 + (size_t)min(sp + u, np - 1) * s.pairs;
      m[u] = p.mpart[at];
      l[u] = sp + u < np ? p.lpart[at] : 0.f;  // a repeated last piece weighs nothing
      const f32x4* src = reinterpret_cast<const f32x4*>(p.opart + at * D + part * DQ);
#pragma unroll
      for (int c = 0; c < NV; ++c) x[u][c] = src[c];
    }
    // Pieces that saw no key of the row (l = 0) weigh nothing.
    float mx = M;
#pragma unroll
    for (int u = 0; u < kMergeAhead; ++u)
      if (l[u] > 0.f) mx = fmaxf(mx, m[u]);
    const float a = M == kNegInf ? 0.f : fast_exp2(M - mx);
    den *= a;
#pragma unroll
    for (int c = 0; c < NV; ++c) num[c] *= a;
#pragma unroll
    for (int u = 0; u < kMergeAhead; ++u) {
      const float wu = l[u] > 0.f ? fast_exp2(m[u] - mx) : 0.f;
      den = fmaf(wu, l[u], den);
#pragma unroll
      for (int c = 0; c < NV; ++c) num[c] += wu * x[u][c];
    }
    M = mx;
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int c = 0; c < DQ / 8; ++c) {
    u32x4 wv;
    wv[0] = pack_bf16x2(num[2 * c][0] * inv, num[2 * c][1] * inv);
    wv[1] = pack_bf16x2(num[2 * c][2] * inv, num[2 * c][3] * inv);
    wv[2] = pack_bf16x2(num[2 * c + 1][0] * inv, num[2 * c + 1][1] * inv);
    wv[3] = pack_bf16x2(num[2 * c + 1][2] * inv, num[2 * c + 1][3] * inv);
    reinterpret_cast<u32x4*>(out)[c] = wv;
  }
  if (part == 0) p.lse[bh * N + row] = (M + __log2f(den)) * kLn2;
}

template <int D, int HP>
hipError_t launch_hp(PrefillParams p, hipStream_t stream) {
  if (p.shape.S <= plan::kMaxRanked)
    hipLaunchKernelGGL(prefill_plan_kernel<true>, dim3(1), dim3(kPlanThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_plan_kernel<false>, dim3(1), dim3(kPlanThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.shape.pairs == 8 * kWQ)
    hipLaunchKernelGGL((prefill_attend_kernel<D, HP, 8>),
                       dim3((unsigned)plan::max_positions(p.shape)), dim3(64 * 8), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_attend_kernel<D, HP, 4>),
                       dim3((unsigned)plan::max_positions(p.shape)), dim3(64 * 4), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_merge_kernel<D, HP>),
                     dim3((unsigned)(plan::max_merge_entries(p.shape) * (p.shape.pairs / kMergePairs))), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(PrefillParams p, int hp, hipStream_t stream) {
  if (hp == 4) return launch_hp<D, 4>(p, stream);
  if (hp == 2) return launch_hp<D, 2>(p, stream);
  return launch_hp<D, 1>(p, stream);
}

}  // namespace

hipError_t launch_paged_prefill(const PagedPrefillArgs& a, hipStream_t stream) {
  PrefillParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k_cache);
  p.v = static_cast<const bf16*>(a.v_cache);
  p.o = static_cast<bf16*>(a.o);
  p.lse = a.lse;
  p.seq_lens = a.seq_lens;
  p.q_lens = a.q_lens;
  p.table = a.block_table;
  p.shape = paged_prefill_shape(a.S, a.max_q, a.Hq, a.Hkv, a.max_blocks);
  const plan::Layout l = plan::layout(p.shape, a.d);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  p.w = plan::bufs(ws, l);
  p.opart = reinterpret_cast<float*>(ws + l.opart);
  p.mpart = reinterpret_cast<float*>(ws + l.mpart);
  p.lpart = reinterpret_cast<float*>(ws + l.lpart);
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.max_blocks = a.max_blocks;
  p.num_blocks = a.num_blocks;
  p.sl2 = a.scale * kLog2e;
  const int hp = p.shape.pairs / p.shape.rph;  // query heads per work item
  return a.d == 128 ? launch_d<128>(p, hp, stream) : launch_d<64>(p, hp, stream);
}

}  // namespace fa
