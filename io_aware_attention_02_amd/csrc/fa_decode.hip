// fa_decode.hip -- decode attention over a paged KV cache (one query token per sequence).
//
// The cache is a pool of physical blocks of 16 tokens, [num_blocks][16][Hkv][d]; a block
// table maps each sequence's logical blocks to physical ones.  Following the non-contiguous
// block gather page (ocdem.com, vLLM PagedAttention rework):
//  * §二.3 -- the block ids a workgroup will visit are loaded into registers up front (one id
//    per lane) and broadcast from there, so no gather waits on the index array;
//  * §二.1 -- each block's keys and values are gathered with coalesced loads (16 lanes cover one
//    256-byte token row) into on-chip memory, then read from there in the layout the matrix
//    cores want (values transposed on the way in);
//  * §二.4 -- gather and attention are one kernel: scores against the register-resident query,
//    online softmax and the probability-weighted sum of values follow each gathered tile.
// Load balance (§二.2 asks for dynamic balancing of unequal per-query work): instead of a
// per-warp task queue, each sequence's tokens are cut into fixed 512-token ranges, one wave
// each, so work per wave is equal whatever the length mix.  Each range writes its partial
// (max, sum, unnormalised output); a second kernel merges them exactly with the rescaling
// rule of the online softmax ("FlashAttention优化" §3.2.2: the result is the same for any
// block order and grouping).
//
// CDNA4 mapping: the Hq/Hkv query heads that share kv head g form the 16 columns of
// v_mfma_f32_16x16x32_bf16 (unused columns are zero).  Scores are S^T = K Q^T (tokens in
// rows, heads in columns); the score accumulator of a lane is already the B operand of
// O^T += V^T P^T, so probabilities stay in registers.  32 tokens (two physical blocks) are
// processed per step; the next step's gathers are in flight while the current one computes.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBS = 16;                         // tokens per physical block
constexpr int kStepTok = 32;                    // tokens per pipeline step (two blocks)
constexpr int kSplit = kDecodeSplitTokens;      // tokens per workgroup
constexpr int kBlocksPerSplit = kSplit / kBS;   // block ids prefetched per workgroup (<= 64)
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
  int Hq, Hkv, group, max_blocks, max_tokens, MS;
  float sl2;
};

template <int D>
struct DTile {
  static constexpr int CPR = D / 8;            // 16-byte chunks per token row
  static constexpr int RPI = 64 / CPR;         // token rows per load instruction
  static constexpr int TPL = kBS / RPI;        // rows per lane per block (consecutive tokens)
  static constexpr int KS = D + 8;             // LDS row stride of K (elements)
  static constexpr int VS = kStepTok + 8;      // LDS row stride of transposed V (elements)
  static constexpr int NB = D / 16;            // 16-dim blocks of the output
  static constexpr int KC = D / 32;            // 32-dim chunks of the score contraction
};

template <int D>
struct DStage {
  u32x4 k[2][DTile<D>::TPL];
  u32x4 v[2][DTile<D>::TPL];
};

// Gather the two blocks of one step into registers.  Lane l covers chunk (l % CPR) of token
// rows TPL*(l / CPR) .. +TPL-1 of each block; tokens at or past L are zero-filled.
template <int D>
__device__ __forceinline__ void gather_step(DStage<D>& st, const DecodeParams& p, int bid0,
                                            int bid1, int tok0, int L, int g, int lane) {
  using T = DTile<D>;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int col = lane % T::CPR, rg = lane / T::CPR;
  const size_t row_stride = (size_t)p.Hkv * D;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    const int bid = bi ? bid1 : bid0;
    const bf16* kb = p.kc + (size_t)bid * kBS * row_stride + (size_t)g * D + col * 8;
    const bf16* vb = p.vc + (size_t)bid * kBS * row_stride + (size_t)g * D + col * 8;
#pragma unroll
    for (int i = 0; i < T::TPL; ++i) {
      const int row = rg * T::TPL + i;
      const bool ok = tok0 + bi * kBS + row < L;
      st.k[bi][i] = ok ? *reinterpret_cast<const u32x4*>(kb + row * row_stride) : zero;
      st.v[bi][i] = ok ? *reinterpret_cast<const u32x4*>(vb + row * row_stride) : zero;
    }
  }
}

// Registers -> LDS.  K keeps [token][dim].  V goes to [dim][position] where token
// 16*bi + 4*h + j sits at position 8*h + 4*bi + j: the k-slot order in which a lane of the
// score accumulator holds its probabilities.
template <int D>
__device__ __forceinline__ void stage_to_lds(const DStage<D>& st, bf16* Ks, bf16* Vt, int lane) {
  using T = DTile<D>;
  const int col = lane % T::CPR, rg = lane / T::CPR;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
    for (int i = 0; i < T::TPL; ++i)
      *reinterpret_cast<u32x4*>(Ks + (bi * kBS + rg * T::TPL + i) * T::KS + col * 8) = st.k[bi][i];
    const int t0 = rg * T::TPL;                      // first token of this lane in the block
    const int pos = 8 * (t0 >> 2) + 4 * bi + (t0 & 3);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int dim = col * 8 + 2 * w;
      if constexpr (T::TPL == 4) {
        const uint32_t x0 = st.v[bi][0][w], x1 = st.v[bi][1][w];
        const uint32_t x2 = st.v[bi][2][w], x3 = st.v[bi][3][w];
        u32x2 lo, hi;
        lo[0] = (x0 & 0xffffu) | (x1 << 16);
        lo[1] = (x2 & 0xffffu) | (x3 << 16);
        hi[0] = (x0 >> 16) | (x1 & 0xffff0000u);
        hi[1] = (x2 >> 16) | (x3 & 0xffff0000u);
        *reinterpret_cast<u32x2*>(Vt + dim * T::VS + pos) = lo;
        *reinterpret_cast<u32x2*>(Vt + (dim + 1) * T::VS + pos) = hi;
      } else {
        static_assert(T::TPL == 2, "head dim 64 or 128");
        const uint32_t x0 = st.v[bi][0][w], x1 = st.v[bi][1][w];
        *reinterpret_cast<uint32_t*>(Vt + dim * T::VS + pos) = (x0 & 0xffffu) | (x1 << 16);
        *reinterpret_cast<uint32_t*>(Vt + (dim + 1) * T::VS + pos) = (x0 >> 16) | (x1 & 0xffff0000u);
      }
    }
  }
}

template <int D>
__global__ void __launch_bounds__(64) decode_split_kernel(DecodeParams p) {
  using T = DTile<D>;
  __shared__ __attribute__((aligned(16))) bf16 Ks[kStepTok * T::KS];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * T::VS];

  const int lane = threadIdx.x;
  const int g = blockIdx.x, sp = blockIdx.y, b = blockIdx.z;
  const int L = min(max(p.lens[b], 0), p.max_tokens);
  const int tok_begin = sp * kSplit;
  if (tok_begin >= L) return;
  const int tok_end = min(L, tok_begin + kSplit);
  const int n_steps = (tok_end - tok_begin + kStepTok - 1) / kStepTok;
  const int blk_begin = tok_begin / kBS;
  const int n_blk = (tok_end - tok_begin + kBS - 1) / kBS;

  // Block ids of this range, one per lane (index prefetch into registers).
  const int my_bid = lane < n_blk ? p.table[(size_t)b * p.max_blocks + blk_begin + lane] : 0;

  // Query fragments: B operand of S^T = K Q^T, column = head (l & 15), k-slots 8*(l >> 4).
  const int head = lane & 15, hq = lane >> 4;
  const bool head_ok = head < p.group;
  const int qh = g * p.group + head;
  bf16x8 qf[T::KC];
#pragma unroll
  for (int c = 0; c < T::KC; ++c) {
    qf[c] = head_ok ? *reinterpret_cast<const bf16x8*>(p.q + ((size_t)b * p.Hq + qh) * D + c * 32 + hq * 8)
                    : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }

  f32x4 acc[T::NB];
#pragma unroll
  for (int n = 0; n < T::NB; ++n) acc[n] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;
  const float sl2 = p.sl2;

  auto bid_at = [&](int i) {  // broadcast block id i of the range (clamped for a tail step)
    return __shfl(my_bid, min(i, n_blk - 1), 64);
  };

  DStage<D> cur, nxt;
  gather_step<D>(cur, p, bid_at(0), bid_at(1), tok_begin, L, g, lane);
  for (int s = 0; s < n_steps; ++s) {
    const int tok0 = tok_begin + s * kStepTok;
    if (s + 1 < n_steps)
      gather_step<D>(nxt, p, bid_at(2 * s + 2), bid_at(2 * s + 3), tok0 + kStepTok, L, g, lane);
    __syncthreads();  // previous step's LDS reads are done
    stage_to_lds<D>(cur, Ks, Vt, lane);
    __syncthreads();

    // Scores for the two blocks: lane holds head (l & 15), tokens 16*bi + 4*(l >> 4) + j.
    f32x4 s2[2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      s2[bi] = f32x4{};
#pragma unroll
      for (int c = 0; c < T::KC; ++c) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (bi * kBS + head) * T::KS + c * 32 + hq * 8);
        s2[bi] = mfma16k32(kf, qf[c], s2[bi]);
      }
    }
    const bool masked = tok0 + kStepTok > L;
    float mx = kNegInf;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (masked && tok0 + bi * kBS + 4 * hq + j >= L) s2[bi][j] = kNegInf;
        mx = fmaxf(mx, s2[bi][j]);
      }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = max_xor32(mx);
    const float mt = (mx == kNegInf) ? kNegInf : mx * sl2;
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float pv[8];
    float rs = 0.f;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = s2[bi][j];
        float e = fast_exp2(fmaf(x, sl2, -m_use));
        if (masked && x == kNegInf) e = 0.f;
        pv[4 * bi + j] = e;
        rs += e;
      }
    l_run = fmaf(alpha, l_run, rs);
    const bf16x8 pf = pack_bf16x8(pv);
#pragma unroll
    for (int n = 0; n < T::NB; ++n) {
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vt + (n * 16 + head) * T::VS + hq * 8);
      acc[n] = mfma16k32(vf, pf, acc[n] * alpha);
    }
    cur = nxt;
  }

  // Partial results of this range: lane (head, hq) holds dims 16*n + 4*hq + j.
  float lt = l_run + shfl_xor(l_run, 16);
  lt = add_xor32(lt);
  if (head_ok) {
    const size_t slot = ((size_t)b * p.Hq + qh) * p.MS + sp;
#pragma unroll
    for (int n = 0; n < T::NB; ++n)
      *reinterpret_cast<f32x4*>(p.opart + slot * D + n * 16 + 4 * hq) = acc[n];
    if (hq == 0) {
      p.mpart[slot] = m_run;
      p.lpart[slot] = lt;
    }
  }
}

// Merge the ranges of one (sequence, query head): M = max m_s, w_s = 2^(m_s - M),
// O = sum w_s O_s / sum w_s l_s, LSE = ln 2 * (M + log2 sum w_s l_s).
template <int D>
__global__ void __launch_bounds__(64) decode_merge_kernel(DecodeParams p) {
  constexpr int DPL = D / 64;  // dims per lane
  const int lane = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = min(max(p.lens[b], 0), p.max_tokens);
  const int n = (L + kSplit - 1) / kSplit;
  const size_t base = ((size_t)b * p.Hq + h) * p.MS;
  bf16* out = p.o + ((size_t)b * p.Hq + h) * D + lane * DPL;
  float M = kNegInf;
  for (int s = 0; s < n; ++s) M = fmaxf(M, p.mpart[base + s]);
  float num[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) num[j] = 0.f;
  float den = 0.f;
  for (int s = 0; s < n; ++s) {
    const float w = fast_exp2(p.mpart[base + s] - M);
    den = fmaf(w, p.lpart[base + s], den);
    const float* src = p.opart + (base + s) * D + lane * DPL;
#pragma unroll
    for (int j = 0; j < DPL; ++j) num[j] = fmaf(w, src[j], num[j]);
  }
  const float inv = n > 0 ? 1.f / den : 0.f;
  if constexpr (DPL == 2) {
    *reinterpret_cast<uint32_t*>(out) = pack_bf16x2(num[0] * inv, num[1] * inv);
  } else {
    out[0] = static_cast<bf16>(num[0] * inv);
  }
  if (p.lse != nullptr && lane == 0)
    p.lse[(size_t)b * p.Hq + h] = n > 0 ? (M + __log2f(den)) * kLn2 : kNegInf;
}

int max_splits(int max_blocks, int block_size) {
  const long long tokens = (long long)max_blocks * block_size;
  return (int)((tokens + kSplit - 1) / kSplit);
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
  p.MS = max_splits(a.max_blocks, a.block_size);
  const size_t slots = (size_t)a.S * a.Hq * p.MS;
  p.opart = static_cast<float*>(a.workspace);
  p.mpart = p.opart + slots * D;
  p.lpart = p.mpart + slots;
  p.sl2 = a.scale * kLog2e;
  hipLaunchKernelGGL(decode_split_kernel<D>, dim3(a.Hkv, p.MS, a.S), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(a.Hq, a.S), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int S, int Hq, int d, int max_blocks, int block_size) {
  if (S <= 0 || Hq <= 0 || d <= 0 || max_blocks <= 0 || block_size <= 0) return 0;
  const size_t slots = (size_t)S * Hq * max_splits(max_blocks, block_size);
  return slots * ((size_t)d + 2) * sizeof(float);
}

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.d == 128 ? launch<128>(a, stream) : launch<64>(a, stream);
}

}  // namespace fa
