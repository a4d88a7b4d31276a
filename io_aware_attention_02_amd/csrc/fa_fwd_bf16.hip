// fa_fwd_bf16.hip -- fused attention forward, bf16 storage, fp32 accumulation, gfx950 MFMA.
//
// One workgroup owns BM query rows of one (batch, head) and streams that head's K/V in tiles
// of BN keys through LDS (the fused, tiled scheme of "Gemini 3 Flash的注意力内核重写" -- kernel
// fusion, tiling -- and "FlashAttention优化" §3.1, with the query block resident and all K/V
// blocks streamed past it).  Per tile it computes scores on the matrix cores, updates the
// running row maximum and row sum with the online-softmax recurrence of "FlashAttention优化"
// §3.2.1, rescales the output accumulator and adds P V on the matrix cores.  Scores and
// probabilities live only in registers.  The output is divided by the row sum once at the
// end (the deferred rescale the "GPU优化" tag page attributes to FlashAttention V2), and the
// natural-log LSE of each row is written beside it.
//
// CDNA4 mapping (not the pages' A100/H100 tile sizes):
//  * Each wave owns 32*QB query rows.  Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K rows (keys) are the A operand read from LDS, Q^T is the B
//    operand held in registers for the whole kernel.  The accumulator then holds one query per
//    lane (lane & 31) and 16 keys per lane, so row max / row sum are mostly in-lane and need
//    one exchange with lane ^ 32 (v_permlane32_swap).  The row sum is kept per half-wave and
//    combined once in the epilogue.
//  * The probabilities of a lane are already the B operand of O^T += V^T P^T (keys in
//    k-slots, query in the lane) after packing to bf16, so P never leaves registers.  V is
//    written to LDS transposed ([dim][key]) with the key order permuted to match the k-slot
//    order of the score accumulator; both contractions then read 16 contiguous bytes per lane.
//  * K/V tiles are double-buffered in LDS: the global loads of tile j+2 are in flight while
//    tile j is computed; tile j+1 goes from registers to the other buffer after it.  One
//    barrier per tile.  LDS rows are padded by 16 bytes so that 16-byte reads of consecutive
//    rows fall in distinct banks.
//  * The grid is one workgroup per (batch, head, query tile), remapped so that the tiles of one
//    head (and of one grouped-query kv head) run on the same XCD and share its L2.  Under
//    causal masking the heaviest query tiles are issued first, tiles past the diagonal are
//    never loaded, and waves whose rows are all above a tile skip it.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <int D, int QB, int NW>
struct Tile {
  static constexpr int BN = 64;             // keys per K/V tile
  static constexpr int WQ = 32 * QB;        // query rows per wave
  static constexpr int BM = WQ * NW;        // query rows per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int KS = D + 8;          // LDS row stride of the K tile (elements)
  static constexpr int VS = BN + 8;         // LDS row stride of the transposed V tile
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  static constexpr int DC = D / 8;          // 16-byte chunks per row
  static constexpr int K_CHUNKS = BN * DC;
  static constexpr int K_ITERS = (K_CHUNKS + THREADS - 1) / THREADS;
  static constexpr int V_UNITS = (BN / 4) * DC;  // 4 keys x 8 dims per unit
  static constexpr int V_ITERS = (V_UNITS + THREADS - 1) / THREADS;
  static constexpr int NB = D / 32;         // 32-dim blocks of the output
  static constexpr int KC = D / 16;         // 16-dim chunks of the score contraction
};

struct Params {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  const int32_t* seq_lens;
  int H, group, Hkv, N, n_qt, total;
  float sl2;  // scale * log2(e): scores go to the exponent base 2
};

template <class T>
struct Stage {
  u32x4 k[T::K_ITERS];
  u32x4 v[T::V_ITERS][4];
};

// Global -> registers for the tile starting at key0.  Keys at or past L are zero-filled, so
// padded or out-of-range rows never reach the arithmetic (not even as NaN * 0).
template <class T, int D>
__device__ __forceinline__ void load_stage(Stage<T>& st, const bf16* Kg, const bf16* Vg, int key0,
                                           int L, int tid) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < T::K_ITERS; ++i) {
    const int c = tid + i * T::THREADS;
    const int row = c / T::DC, col = c % T::DC;
    const int key = key0 + row;
    st.k[i] = (c < T::K_CHUNKS && key < L)
                  ? *reinterpret_cast<const u32x4*>(Kg + (size_t)key * D + col * 8)
                  : zero;
  }
#pragma unroll
  for (int i = 0; i < T::V_ITERS; ++i) {
    const int u = tid + i * T::THREADS;
    const int quad = u / T::DC, col = u % T::DC;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + quad * 4 + r;
      st.v[i][r] = (u < T::V_UNITS && key < L)
                       ? *reinterpret_cast<const u32x4*>(Vg + (size_t)key * D + col * 8)
                       : zero;
    }
  }
}

// Registers -> LDS.  K keeps its [key][dim] layout.  V is transposed to [dim][key]: each unit
// of 4 keys x 8 dims becomes 8 runs of 4 keys.  Inside every 16-key group the two middle
// quads swap places (key quad q goes to position quad ((q & 1) << 1) | (q >> 1)), which is
// the k-slot order of the score accumulator: lane half 0 holds keys {0-3, 8-11} of the group,
// half 1 keys {4-7, 12-15}.
template <class T>
__device__ __forceinline__ void store_stage(const Stage<T>& st, bf16* buf, int tid) {
  bf16* Ks = buf;
  bf16* Vt = buf + T::K_ELEMS;
#pragma unroll
  for (int i = 0; i < T::K_ITERS; ++i) {
    const int c = tid + i * T::THREADS;
    if (c < T::K_CHUNKS) {
      const int row = c / T::DC, col = c % T::DC;
      *reinterpret_cast<u32x4*>(Ks + row * T::KS + col * 8) = st.k[i];
    }
  }
#pragma unroll
  for (int i = 0; i < T::V_ITERS; ++i) {
    const int u = tid + i * T::THREADS;
    if (u < T::V_UNITS) {
      const int quad = u / T::DC, col = u % T::DC;
      const int qg = quad & 3;
      const int pos = (quad >> 2) * 16 + ((((qg & 1) << 1) | (qg >> 1)) << 2);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x0 = st.v[i][0][w], x1 = st.v[i][1][w];
        const uint32_t x2 = st.v[i][2][w], x3 = st.v[i][3][w];
        u32x2 lo, hi;  // dims 2w and 2w+1, keys 0..3 of the quad
        lo[0] = (x0 & 0xffffu) | (x1 << 16);
        lo[1] = (x2 & 0xffffu) | (x3 << 16);
        hi[0] = (x0 >> 16) | (x1 & 0xffff0000u);
        hi[1] = (x2 >> 16) | (x3 & 0xffff0000u);
        const int dim = col * 8 + 2 * w;
        *reinterpret_cast<u32x2*>(Vt + dim * T::VS + pos) = lo;
        *reinterpret_cast<u32x2*>(Vt + (dim + 1) * T::VS + pos) = hi;
      }
    }
  }
}

template <int D, bool CAUSAL, int QB, int NW>
__global__ void __launch_bounds__(64 * NW) fwd_bf16_kernel(Params p) {
  using T = Tile<D, QB, NW>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * T::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, hh = lane >> 5;

  const int lam = xcd_remap(blockIdx.x, p.total);
  const int bh = lam / p.n_qt;
  int qt = lam - bh * p.n_qt;
  if (CAUSAL) qt = p.n_qt - 1 - qt;  // heaviest query tiles first
  const int H = p.H, N = p.N;
  const int b = bh / H, h = bh - b * H;
  const int g = h / p.group;
  int L = N;
  if (p.seq_lens != nullptr) L = min(max(p.seq_lens[b], 0), N);

  const int q0 = qt * T::BM;
  const bf16* Qg = p.q + (size_t)bh * N * D;
  const bf16* Kg = p.k + (size_t)(b * p.Hkv + g) * N * D;
  const bf16* Vg = p.v + (size_t)(b * p.Hkv + g) * N * D;
  bf16* Og = p.o + (size_t)bh * N * D;
  float* LSEg = p.lse + (size_t)bh * N;

  if (q0 >= L) {  // every row of this tile is padding: O = 0, LSE = -inf
    const int rows = min(T::BM, N - q0);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int i = tid; i < rows * T::DC; i += T::THREADS)
      *reinterpret_cast<u32x4*>(Og + (size_t)q0 * D + i * 8) = zero;
    for (int r = tid; r < rows; r += T::THREADS) LSEg[q0 + r] = kNegInf;
    return;
  }

  const int kv_end = CAUSAL ? min(L, q0 + T::BM) : L;
  const int n_kt = (kv_end + T::BN - 1) / T::BN;
  const int qw0 = q0 + wave * T::WQ;
  const float sl2 = p.sl2;

  // Q^T fragments (B operand of S^T = K Q^T), resident for the whole kernel.
  bf16x8 qf[QB][T::KC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + c32;
#pragma unroll
    for (int c = 0; c < T::KC; ++c) {
      if (row < N) {
        qf[qb][c] = *reinterpret_cast<const bf16x8*>(Qg + (size_t)row * D + c * 16 + hh * 8);
      } else {
        qf[qb][c] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      }
    }
  }

  float m_run[QB], l_run[QB];
  f32x16 acc[T::NB][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
#pragma unroll
    for (int n = 0; n < T::NB; ++n) acc[n][qb] = f32x16{};
  }

  Stage<T> st;
  load_stage<T, D>(st, Kg, Vg, 0, L, tid);
  store_stage<T>(st, smem, tid);
  __syncthreads();
  if (n_kt > 1) load_stage<T, D>(st, Kg, Vg, T::BN, L, tid);

  for (int kt = 0; kt < n_kt; ++kt) {
    const int key0 = kt * T::BN;
    const bf16* Ks = smem + (kt & 1) * T::BUF;
    const bf16* Vt = Ks + T::K_ELEMS;
    if (!CAUSAL || key0 <= qw0 + T::WQ - 1) {
      const bool masked = (key0 + T::BN > L) || (CAUSAL && key0 + T::BN - 1 > qw0);

      // S^T[key][query] for the 64 keys of the tile (two 32-key blocks).
      f32x16 s[2][QB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
      for (int c = 0; c < T::KC; ++c) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + c32) * T::KS + c * 16 + hh * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32(kf, qf[qb][c], s[kb][qb]);
        }
      }

      // Online softmax: running max m (base-2 exponent units), running sum l, rescale.
      bf16x8 pf[QB][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (masked) {
          const int qrow = qw0 + qb * 32 + c32;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
              const bool ok = key < L && (!CAUSAL || key <= qrow);
              if (!ok) s[kb][qb][r] = kNegInf;
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
        mx = max_xor32(mx);
        const float mt = (mx == kNegInf) ? kNegInf : mx * sl2;
        const float m_new = fmaxf(m_run[qb], mt);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run[qb] - m_use);
        m_run[qb] = m_new;
        float pv[32];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float x = s[kb][qb][r];
            float e = fast_exp2(fmaf(x, sl2, -m_use));
            if (masked && x == kNegInf) e = 0.f;
            pv[kb * 16 + r] = e;
            rs += e;
          }
        l_run[qb] = fmaf(alpha, l_run[qb], rs);
#pragma unroll
        for (int n = 0; n < T::NB; ++n) acc[n][qb] *= alpha;
#pragma unroll
        for (int j = 0; j < 4; ++j) pf[qb][j] = pack_bf16x8(&pv[8 * j]);
      }

      // O^T[dim][query] += V^T[dim][key] P^T[key][query].
#pragma unroll
      for (int n = 0; n < T::NB; ++n) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8*>(Vt + (n * 32 + c32) * T::VS + j * 16 + hh * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[n][qb] = mfma32(vf, pf[qb][j], acc[n][qb]);
        }
      }
    }
    if (kt + 1 < n_kt) {
      store_stage<T>(st, smem + ((kt + 1) & 1) * T::BUF, tid);
      if (kt + 2 < n_kt) load_stage<T, D>(st, Kg, Vg, (kt + 2) * T::BN, L, tid);
    }
    __syncthreads();
  }

  // Epilogue: O = acc / l once; LSE = ln 2 * (m + log2 l).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = add_xor32(l_run[qb]);
    const int row = qw0 + qb * 32 + c32;
    if (row < N) {
      const bool valid = row < L;
      const float inv = valid ? 1.f / lt : 0.f;
#pragma unroll
      for (int n = 0; n < T::NB; ++n) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float x[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) x[j] = valid ? acc[n][qb][4 * r4 + j] * inv : 0.f;
          u32x2 w;
          w[0] = pack_bf16x2(x[0], x[1]);
          w[1] = pack_bf16x2(x[2], x[3]);
          *reinterpret_cast<u32x2*>(Og + (size_t)row * D + n * 32 + 8 * r4 + 4 * hh) = w;
        }
      }
      if (hh == 0) LSEg[row] = valid ? (m_run[qb] + __log2f(lt)) * kLn2 : kNegInf;
    }
  }
}

// Tile shape chosen for gfx950: 4 waves x 32 query rows, 64-key tiles, ~70 KB of LDS per
// workgroup (two workgroups fit in a CU's 160 KB).
constexpr int kQB = 1;
constexpr int kNW = 4;

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  using T = Tile<D, kQB, kNW>;
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
  p.n_qt = (a.N + T::BM - 1) / T::BM;
  p.total = a.B * a.H * p.n_qt;
  p.sl2 = a.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, kQB, kNW>), dim3(p.total), dim3(T::THREADS), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

int fwd_bf16_rows_per_workgroup() { return Tile<128, kQB, kNW>::BM; }

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
