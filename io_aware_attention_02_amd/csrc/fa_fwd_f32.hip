// fa_fwd_f32.hip -- fused attention forward with fp32 storage and fp32 arithmetic.
//
// Same method as the bf16 kernel -- K/V streamed through LDS in tiles, scores and
// probabilities kept on chip, running max / running sum with rescaling ("FlashAttention优化"
// §3.1 and §3.2.1), one division by the row sum at the end, natural-log LSE per row -- but
// every product and sum is an fp32 FMA on the vector ALUs.  One lane owns one query row: it
// holds its query and its output accumulator in registers and reads each key and value row
// of the tile from LDS as a broadcast.  This variant exists for accuracy (fp32 end to end);
// the bf16 kernel is the throughput path.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 128;  // query rows per workgroup
constexpr int kBN = 32;        // keys per tile

struct ParamsF32 {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  const int32_t* seq_lens;
  int H, group, Hkv, N, n_qt, total;
  float sl2;
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) fwd_f32_kernel(ParamsF32 p) {
  __shared__ __attribute__((aligned(16))) float Ks[kBN][D];
  __shared__ __attribute__((aligned(16))) float Vs[kBN][D];

  const int tid = threadIdx.x;
  const int lam = xcd_remap(blockIdx.x, p.total);
  const int bh = lam / p.n_qt;
  int qt = lam - bh * p.n_qt;
  if (CAUSAL) qt = p.n_qt - 1 - qt;
  const int N = p.N;
  const int b = bh / p.H, h = bh - b * p.H;
  const int g = h / p.group;
  int L = N;
  if (p.seq_lens != nullptr) L = min(max(p.seq_lens[b], 0), N);

  const int q0 = qt * kThreads;
  const int row = q0 + tid;
  const float* Qg = p.q + (size_t)bh * N * D;
  const float* Kg = p.k + (size_t)(b * p.Hkv + g) * N * D;
  const float* Vg = p.v + (size_t)(b * p.Hkv + g) * N * D;
  float* Og = p.o + (size_t)bh * N * D;
  float* LSEg = p.lse + (size_t)bh * N;

  if (q0 >= L) {  // padding tile
    if (row < N) {
      for (int c = 0; c < D; c += 4) *reinterpret_cast<f32x4*>(Og + (size_t)row * D + c) = f32x4{};
      LSEg[row] = kNegInf;
    }
    return;
  }

  float qr[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    f32x4 x = f32x4{};
    if (row < N) x = *reinterpret_cast<const f32x4*>(Qg + (size_t)row * D + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qr[c + j] = x[j];
      acc[c + j] = 0.f;
    }
  }
  float m_run = kNegInf, l_run = 0.f;
  const float sl2 = p.sl2;
  const int kv_end = CAUSAL ? min(L, q0 + kThreads) : L;
  const int n_kt = (kv_end + kBN - 1) / kBN;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int key0 = kt * kBN;
    __syncthreads();  // previous tile fully consumed
    for (int i = tid; i < kBN * D / 4; i += kThreads) {
      const int r = i / (D / 4), c = (i % (D / 4)) * 4;
      const int key = key0 + r;
      f32x4 kx = f32x4{}, vx = f32x4{};
      if (key < L) {
        kx = *reinterpret_cast<const f32x4*>(Kg + (size_t)key * D + c);
        vx = *reinterpret_cast<const f32x4*>(Vg + (size_t)key * D + c);
      }
      *reinterpret_cast<f32x4*>(&Ks[r][c]) = kx;
      *reinterpret_cast<f32x4*>(&Vs[r][c]) = vx;
    }
    __syncthreads();

    float s[kBN];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      float d0 = 0.f, d1 = 0.f;
#pragma unroll
      for (int c = 0; c < D; c += 2) {
        d0 = fmaf(qr[c], Ks[j][c], d0);
        d1 = fmaf(qr[c + 1], Ks[j][c + 1], d1);
      }
      const int key = key0 + j;
      const bool ok = key < L && (!CAUSAL || key <= row);
      s[j] = ok ? d0 + d1 : kNegInf;
      mx = fmaxf(mx, s[j]);
    }
    const float mt = (mx == kNegInf) ? kNegInf : mx * sl2;
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      const float e = (s[j] == kNegInf) ? 0.f : exp2f(fmaf(s[j], sl2, -m_use));
      s[j] = e;
      rs += e;
    }
    l_run = fmaf(alpha, l_run, rs);
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      const float e = s[j];
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(e, Vs[j][c], acc[c]);
    }
  }

  if (row < N) {
    const bool valid = row < L;
    const float inv = valid ? 1.f / l_run : 0.f;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      f32x4 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = valid ? acc[c + j] * inv : 0.f;
      *reinterpret_cast<f32x4*>(Og + (size_t)row * D + c) = x;
    }
    LSEg[row] = valid ? (m_run + log2f(l_run)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  ParamsF32 p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.o = static_cast<float*>(a.o);
  p.lse = a.lse;
  p.seq_lens = a.seq_lens;
  p.H = a.H;
  p.group = a.H / a.Hkv;
  p.Hkv = a.Hkv;
  p.N = a.N;
  p.n_qt = (a.N + kThreads - 1) / kThreads;
  p.total = a.B * a.H * p.n_qt;
  p.sl2 = a.scale * kLog2e;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(p.total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
