// Fused attention forward with float32 tensors and fp32 arithmetic throughout (gfx950).
//
// Same method as the bf16 kernel -- the FlashAttention-2 recurrence of "FlashAttention-2: Faster
// Attention with Better Parallelism and Work Partitioning" (section "방법론 / 알고리즘 개요"): K/V
// blocks streamed through LDS, running max and sum, rescaled accumulator, one final 1/l, blocks
// above the causal diagonal skipped.  There is no fp32 matrix-core path here: this instance
// exists for fp32 inputs, where exactness matters more than speed, so the products run on the
// vector ALUs.  Four lanes share one query row (each owns a quarter of the head dimension) and
// combine their partial dot products with two lane swaps.
#include "fa_device.h"
#include "fa_kernels.h"

#include <math.h>

namespace fa {
namespace {

constexpr int F32_ROWS = 64;   // query rows per workgroup
constexpr int F32_BC = 32;     // keys per K/V block
constexpr int F32_NT = 256;    // threads: 4 per query row

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, float scale,
    float scale_log2) {
  constexpr int DQ = D / 4;  // head-dim elements per lane
  __shared__ float ks[F32_BC][D + 4];
  __shared__ float vs[F32_BC][D + 4];

  const int tid = threadIdx.x;
  const int row = tid >> 2, part = tid & 3;
  const int hq = blockIdx.y, b = blockIdx.z;
  const int hkv = hq / (Hq / Hkv);
  const int q0 = blockIdx.x * F32_ROWS;
  const int my_q = q0 + row;
  const int off = Nk - Nq;
  const size_t bh = (size_t)b * Hq + hq;

  float qv[DQ], acc[DQ];
  const float* qrow = Q + (bh * Nq + my_q) * D + part * DQ;
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    qv[e] = my_q < Nq ? qrow[e] : 0.f;
    acc[e] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(Nq - 1, q0 + F32_ROWS - 1) + off + 1);
  const float* Kh = K + ((size_t)b * Hkv + hkv) * Nk * D;
  const float* Vh = V + ((size_t)b * Hkv + hkv) * Nk * D;
  const int lim = CAUSAL ? min(Nk - 1, my_q + off) : Nk - 1;

  for (int k0 = 0; k0 < kv_end; k0 += F32_BC) {
    __syncthreads();
    for (int i = tid; i < F32_BC * D; i += F32_NT) {
      const int r = i / D, c = i - r * D;
      const int key = k0 + r;
      ks[r][c] = key < Nk ? Kh[(size_t)key * D + c] : 0.f;
      vs[r][c] = key < Nk ? Vh[(size_t)key * D + c] : 0.f;
    }
    __syncthreads();

    float s[F32_BC];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < F32_BC; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) dot = fmaf(qv[e], ks[j][part * DQ + e], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      s[j] = (k0 + j <= lim) ? dot : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * scale_log2);
    const float mb = m_use * scale_log2;
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < DQ; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < F32_BC; ++j) {
      const float p = fast_exp2(fmaf(s[j], scale_log2, -mb));
      rs += p;
#pragma unroll
      for (int e = 0; e < DQ; ++e) acc[e] = fmaf(p, vs[j][part * DQ + e], acc[e]);
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
  }

  if (my_q < Nq) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* orow = O + (bh * Nq + my_q) * D + part * DQ;
#pragma unroll
    for (int e = 0; e < DQ; ++e) orow[e] = acc[e] * inv;
    if (LSE != nullptr && part == 0)
      LSE[bh * Nq + my_q] = l_run > 0.f ? m_run * scale + logf(l_run) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const float* q, const float* k, const float* v, float* out, float* lse,
                  const AttnShape& s, float scale, hipStream_t stream) {
  const dim3 grid((s.Nq + F32_ROWS - 1) / F32_ROWS, s.Hq, s.B);
  if (grid.y > 65535u || grid.z > 65535u) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), grid, dim3(F32_NT), 0, stream, q, k, v, out,
                     lse, s.Hq, s.Hkv, s.Nq, s.Nk, scale, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* out,
                          float* lse, const AttnShape& s, float scale, bool causal,
                          hipStream_t stream) {
  if (s.d == 128)
    return causal ? launch<128, true>(q, k, v, out, lse, s, scale, stream)
                  : launch<128, false>(q, k, v, out, lse, s, scale, stream);
  return causal ? launch<64, true>(q, k, v, out, lse, s, scale, stream)
                : launch<64, false>(q, k, v, out, lse, s, scale, stream);
}

}  // namespace fa
