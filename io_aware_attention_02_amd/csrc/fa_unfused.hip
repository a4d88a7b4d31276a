// fa_unfused.hip -- the standard, unfused attention forward, as a baseline for the fused kernel.
//
// "FlashAttention优化" §2.1-§2.2 and "Gemini 3 Flash的注意力内核重写" (the section on the memory
// bottleneck of standard attention) describe the implementation that fusion replaces: the
// score matrix S = scale * Q K^T is written to device memory, a softmax pass reads it (three
// passes over each row: maximum, sum of exponentials, normalisation) and writes P, and a third
// kernel reads P to form O = P V.  These kernels do exactly that on the same matrix-core tiles
// as the fused kernel, so the measured difference is the cost of the N x N round trips.
//
//  * unf_scores_kernel   S (fp32, [B, H, N, N] row-major), one workgroup per (b, h, 128 rows);
//                        under causal masking only tiles that reach the diagonal are computed
//                        (entries past a row's last visible key are never read).
//  * unf_softmax_kernel  one wave per row: max, sum of exp(s - max), then P = exp(s - max) / sum
//                        in bf16 ([B, H, N, N], zero past the last visible key) and LSE.
//  * unf_pv_kernel       O = P V: P fragments straight from device memory in the matrix-core
//                        B-operand order, V tiles through LDS (transposing reads).
#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tiles.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kNWu = 4;  // waves per workgroup of the two matrix kernels

struct UnfParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  float* s;  // [B, H, N, N]
  bf16* p;   // [B, H, N, N]
  int H, group, Hkv, N, n_qt;
  float scale;
};

// S^T tiles of 64 keys x 32 queries per wave, stored row-major as S[query][key]: the
// accumulator lane (query c32, half hh) holds keys 8*(r>>2) + 4*hh + (r&3), i.e. four runs of
// four consecutive keys per 32-key block.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * kNWu) __attribute__((amdgpu_waves_per_eu(2, 2)))
unf_scores_kernel(UnfParams p) {
  using G = Geo<D>;
  constexpr int NW = kNWu;
  constexpr int kBM = NW * kWQ;
  constexpr int NI_W = LoadGeo<D, NW>::NI_W;
  __shared__ __attribute__((aligned(1024))) char k0s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[G::TILE];
  lds_t* const K0 = (lds_t*)k0s;
  lds_t* const K1 = (lds_t*)k1s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c32 = lane & 31, hh = lane >> 5;
  const int bh = blockIdx.x / p.n_qt, qt = blockIdx.x - bh * p.n_qt;
  const int N = p.N;
  const int b = bh / p.H, h = bh - b * p.H, g = h / p.group;
  const int q0 = qt * kBM, qrow = q0 + wave * kWQ + c32;
  const bf16* Qg = p.q + (size_t)bh * N * D;
  const bf16* Kg = p.k + (size_t)(b * p.Hkv + g) * N * D;
  float* Sg = p.s + (size_t)bh * N * N;
  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int n_kt = (kv_end + kBN - 1) / kBN;
  int off[NI_W];
  tile_offsets<D, NW, false>(off, wave, lane);
  load_tile<D, NW>(K0, Kg, 0, N, off, wave);
  bf16x8 qf[G::KC];
#pragma unroll
  for (int c = 0; c < G::KC; ++c)
    qf[c] = qrow < N ? *reinterpret_cast<const bf16x8*>(Qg + (size_t)qrow * D + c * 16 + hh * 8)
                     : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  const FragAddr<D> fa = frag_addr<D>(lane);
  f32x16 sA[2];
  wait_loads();
  __syncthreads();
  for (int j = 0; j < n_kt; ++j) {
    lds_t* const Kc = (j & 1) ? K1 : K0;
    lds_t* const Kn = (j & 1) ? K0 : K1;
    if (j + 1 < n_kt) load_tile<D, NW>(Kn, Kg, (j + 1) * kBN, N, off, wave);
    scores<D>(sA, Kc, fa, qf);
    if (qrow < N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int key = j * kBN + kb * 32 + 8 * r4 + 4 * hh;
          if (key < N) {  // N is a multiple of 4 or the last run is partial
            f32x4 w;
#pragma unroll
            for (int t = 0; t < 4; ++t) w[t] = sA[kb][4 * r4 + t] * p.scale;
            if (key + 4 <= N) {
              *reinterpret_cast<f32x4*>(Sg + (size_t)qrow * N + key) = w;
            } else {
              for (int t = 0; key + t < N; ++t) Sg[(size_t)qrow * N + key + t] = w[t];
            }
          }
        }
    }
    wait_loads();
    __syncthreads();
  }
}

// One wave per row: three passes over the row's visible scores, as the unfused standard
// implementation does.
__global__ void __launch_bounds__(256) unf_softmax_kernel(UnfParams p, int causal, long long rows) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int N = p.N;
  const int i = (int)(row % N);
  const int count = causal ? i + 1 : N;
  const float* S = p.s + row * N;
  bf16* P = p.p + row * N;
  // pass 1: row maximum
  float m = kNegInf;
  for (int j = lane; j < count; j += 64) m = fmaxf(m, S[j]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  // pass 2: sum of exponentials relative to the maximum
  float l = 0.f;
  for (int j = lane; j < count; j += 64) l += fast_exp2((S[j] - m) * kLog2e);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
  // pass 3: normalise (zero past the last visible key) and the row's LSE
  const float inv = 1.f / l;
  for (int j = lane; j < N; j += 64) {
    const float e = j < count ? fast_exp2((S[j] - m) * kLog2e) * inv : 0.f;
    P[j] = static_cast<bf16>(e);
  }
  if (lane == 0) p.lse[row] = m + __logf(l);
}

// O^T (d x 32 queries per wave) = V^T P^T over key tiles of 64; P read from device memory in
// the B-operand order of the fused kernel's probabilities (keys 16 jj + 4 hh + {0..3} and
// 16 jj + 8 + 4 hh + {0..3} for chunk jj).
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * kNWu) __attribute__((amdgpu_waves_per_eu(2, 2)))
unf_pv_kernel(UnfParams p) {
  using G = Geo<D>;
  constexpr int NW = kNWu;
  constexpr int kBM = NW * kWQ;
  constexpr int NI_W = LoadGeo<D, NW>::NI_W;
  __shared__ __attribute__((aligned(1024))) char v0s[G::TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[G::TILE];
  lds_t* const V0 = (lds_t*)v0s;
  lds_t* const V1 = (lds_t*)v1s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c32 = lane & 31, hh = lane >> 5;
  const int bh = blockIdx.x / p.n_qt, qt = blockIdx.x - bh * p.n_qt;
  const int N = p.N;
  const int b = bh / p.H, h = bh - b * p.H, g = h / p.group;
  const int q0 = qt * kBM, qw0 = q0 + wave * kWQ, qrow = qw0 + c32;
  const bf16* Vg = p.v + (size_t)(b * p.Hkv + g) * N * D;
  const bf16* Pg = p.p + (size_t)bh * N * N + (size_t)min(qrow, N - 1) * N;
  bf16* Og = p.o + (size_t)bh * N * D;
  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int n_kt = (kv_end + kBN - 1) / kBN;
  const int n_kw = CAUSAL ? min(n_kt, (min(N, qw0 + kWQ) + kBN - 1) / kBN) : n_kt;
  int off[NI_W];
  tile_offsets<D, NW, true>(off, wave, lane);
  load_tile<D, NW>(V0, Vg, 0, N, off, wave);
  const FragAddr<D> fa = frag_addr<D>(lane);
  f32x16 acc[G::NB];
#pragma unroll
  for (int n = 0; n < G::NB; ++n) acc[n] = f32x16{};
  wait_loads();
  __syncthreads();
  for (int j = 0; j < n_kt; ++j) {
    lds_t* const Vc = (j & 1) ? V1 : V0;
    lds_t* const Vn = (j & 1) ? V0 : V1;
    if (j + 1 < n_kt) load_tile<D, NW>(Vn, Vg, (j + 1) * kBN, N, off, wave);
    if (j < n_kw) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int k0 = j * kBN + 16 * jj + 4 * hh;
        u32x2 lo = {0u, 0u}, hi = {0u, 0u};
        if (qrow < N && k0 + 4 <= N) lo = *reinterpret_cast<const u32x2*>(Pg + k0);
        if (qrow < N && k0 + 12 <= N) hi = *reinterpret_cast<const u32x2*>(Pg + k0 + 8);
        const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int n = 0; n < G::NB; ++n) {
          const lds_t* vp = Vc + fa.v[n] + jj * 16 * G::RB;
          const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)vp);
          const i16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 8 * G::RB));
          acc[n] = mfma32(__builtin_bit_cast(bf16x8, __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7)),
                          pf, acc[n]);
        }
      }
    }
    wait_loads();
    __syncthreads();
  }
  if (qrow < N) {
#pragma unroll
    for (int n = 0; n < G::NB; ++n)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[n][4 * r4 + 0], acc[n][4 * r4 + 1]);
        w[1] = pack_bf16x2(acc[n][4 * r4 + 2], acc[n][4 * r4 + 3]);
        *reinterpret_cast<u32x2*>(Og + (size_t)qrow * D + n * 32 + 8 * r4 + 4 * hh) = w;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const UnfusedArgs& a, hipStream_t stream) {
  UnfParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.o = static_cast<bf16*>(a.o);
  p.lse = a.lse;
  p.s = static_cast<float*>(a.workspace);
  p.p = reinterpret_cast<bf16*>(static_cast<char*>(a.workspace) +
                                (size_t)a.B * a.H * a.N * a.N * sizeof(float));
  p.H = a.H;
  p.group = a.H / a.Hkv;
  p.Hkv = a.Hkv;
  p.N = a.N;
  p.n_qt = (a.N + kNWu * kWQ - 1) / (kNWu * kWQ);
  p.scale = a.scale;
  const unsigned grid = (unsigned)(a.B * a.H * p.n_qt);
  hipLaunchKernelGGL((unf_scores_kernel<D, CAUSAL>), dim3(grid), dim3(64 * kNWu), 0, stream, p);
  const long long rows = (long long)a.B * a.H * a.N;
  hipLaunchKernelGGL(unf_softmax_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, p,
                     CAUSAL ? 1 : 0, rows);
  hipLaunchKernelGGL((unf_pv_kernel<D, CAUSAL>), dim3(grid), dim3(64 * kNWu), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_unfused(const UnfusedArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
