// Split-KV decode attention for gfx950: a fused split kernel and a combine kernel.
//
// Method: "[onnxruntime] WebGPU FlashAttention 최적화: 커널 퓨전과 가변 시퀀스 길이 지원으로 성능
// 극대화".  Section 1 (kernel fusion): one program computes QKᵀ, the causal mask, a local softmax,
// the normalisation and the product with V for its slice of the keys, and writes a partial output
// plus (local max, local sum) metadata; a reduce step rescales the locally normalised partials so
// that their combination is exactly softmax(QKᵀ)·V.  Section 2: each workgroup serves several query
// rows so that the K/V it streams is read once for all of them.
//
// gfx950 mapping:
//   * split kernel: one workgroup (4 waves) per (batch, KV head, row group of 32, split).  The
//     32 "query" columns of the MFMA are the Hq/Hkv query heads x Nq rows that share the KV head,
//     so every K/V byte of the split is read from HBM exactly once.  Each wave streams its own
//     32-key blocks (block w, w+4, ...) through a wave-private LDS slice with 16-byte coalesced
//     loads, prefetching its next block while it computes, and keeps its own running (m, l, Oᵀ);
//     the 4 waves are merged through LDS at the end into one locally normalised partial.
//   * The products use v_mfma_f32_32x32x16_bf16 exactly as the prefill kernel does: Sᵀ = K·Qᵀ,
//     Oᵀ += Vᵀ·Pᵀ with Vᵀ from the transposing LDS read.
//   * combine kernel: one wave per (batch, query head, row); the split metadata is read by all
//     lanes at once and the partial rows are accumulated in a fixed split order, so the result
//     is deterministic.
#include "fa_device.h"
#include "fa_kernels.h"

#include <math.h>

namespace fa {
namespace {

template <int D>
struct DecCfg {
  static constexpr int KB = 32;               // keys per wave block
  static constexpr int NW = 4;                // waves per workgroup
  static constexpr int NT = 64 * NW;
  // LDS pitches (bf16), each conflict-free for its read pattern on gfx950's 64 x 4-byte banks:
  // K rows read 16 bytes per lane (pad 16 bytes), V rows read by transposing 8-byte reads
  // (pad 64 bytes).
  static constexpr int KROW = D + 8;
  static constexpr int VROW = D + 32;
  static constexpr int WTILE = KB * (KROW + VROW);  // one wave's K block + V block (bf16)
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int NCH = KB * CPR / 64;   // chunks per lane per tensor
  static constexpr int OROW = D + 4;          // fp32 pitch of the cross-wave merge buffer
  static constexpr int STAGE_BYTES = NW * WTILE * 2;
  static constexpr int MERGE_BYTES = NW * 32 * OROW * 4 + NW * 32 * 3 * 4;
  static constexpr int SMEM = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
};

// Orders this wave's LDS writes before its later LDS reads of other lanes' data.  A wave's LDS
// operations complete in issue order, so only compiler reordering has to be prevented.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ wsO, float* __restrict__ wsML, int Hq,
    int Hkv, int Nq, int Nk, int S, int L, int nrg, float scale, float scale_log2) {
  using C = DecCfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  int n = blockIdx.x;
  const int s = n % S;
  n /= S;
  const int rg = n % nrg;
  n /= nrg;
  const int hkv = n % Hkv, b = n / Hkv;
  const int G = Hq / Hkv, R = G * Nq;
  const int off = Nk - Nq;

  // this lane's query column: row r of the KV head's group = (query head offset g, position qi)
  const int r = rg * 32 + l32;
  const bool row_ok = r < R;
  const int g = row_ok ? r / Nq : 0;
  const int qi = row_ok ? r - g * Nq : 0;
  const int hq = hkv * G + g;

  const int ks0 = min(s * L, Nk), ks1 = min(ks0 + L, Nk);
  const int nkb = (ks1 - ks0 + C::KB - 1) / C::KB;
  const int lim = CAUSAL ? min(ks1 - 1, qi + off) : ks1 - 1;  // last visible key of this row

  u32x4 qf[D / 16];
  {
    const uint16_t* qrow = Q + (((size_t)b * Hq + hq) * Nq + qi) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qf[c] = row_ok ? *(const u32x4*)(qrow + 16 * c + 8 * h) : u32x4{0u, 0u, 0u, 0u};
  }

  const uint16_t* Kh = K + ((size_t)b * Hkv + hkv) * Nk * D;
  const uint16_t* Vh = V + ((size_t)b * Hkv + hkv) * Nk * D;
  uint16_t* kls = (uint16_t*)smem + wave * C::WTILE;
  uint16_t* vls = kls + C::KB * C::KROW;

  u32x4 kst[C::NCH], vst[C::NCH];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < C::NCH; ++i) {
      const int ci = lane + 64 * i;
      const int row = ci / C::CPR, col = (ci % C::CPR) * 8;
      const int key = ks0 + C::KB * kb + row;
      if (key < ks1) {  // keys of the next split or past Nk are not this split's: zero
        kst[i] = *(const u32x4*)(Kh + (size_t)key * D + col);
        vst[i] = *(const u32x4*)(Vh + (size_t)key * D + col);
      } else {
        kst[i] = u32x4{0u, 0u, 0u, 0u};
        vst[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto swrite = [&]() {
#pragma unroll
    for (int i = 0; i < C::NCH; ++i) {
      const int ci = lane + 64 * i;
      const int row = ci / C::CPR, col = (ci % C::CPR) * 8;
      *(u32x4*)(kls + row * C::KROW + col) = kst[i];
      *(u32x4*)(vls + row * C::VROW + col) = vst[i];
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  // m_run: the lazily moved reference the exponents use; m_true: the exact running max, which
  // the stored metadata reports
  float m_run = -INFINITY, m_true = -INFINITY, l_run = 0.f;
  const int tr_g = lane >> 4, tr_j = (lane & 15) >> 2, tr_t = lane & 3;

  int kb = wave;
  if (kb < nkb) gload(kb);
  for (; kb < nkb; kb += C::NW) {
    swrite();
    wave_lds_sync();
    if (kb + C::NW < nkb) gload(kb + C::NW);  // in flight while this block is computed
    const int k0 = ks0 + C::KB * kb;

    f32x16 sc = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const u32x4 a = *(const u32x4*)(kls + l32 * C::KROW + 16 * c + 8 * h);
      sc = mfma32x32x16(a, qf[c], sc);
    }
    if (k0 + C::KB - 1 > lim || (CAUSAL && k0 + C::KB - 1 > off)) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = k0 + 8 * (rr >> 2) + 4 * h + (rr & 3);
        if (key > lim) sc[rr] = -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int rr = 1; rr < 16; ++rr) mx = fmaxf(mx, sc[rr]);
    mx = pair32_max(mx);
    m_true = fmaxf(m_true, mx);
    const bool grow = (mx - m_run) * scale_log2 > kLazyLog2;  // lazy reference max, as in prefill
    const float m_next = grow ? mx : m_run;
    const float alpha = grow ? fast_exp2((m_run - m_next) * scale_log2) : 1.f;
    if (wave_any(grow && m_run != -INFINITY)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    m_run = m_next;
    const float mb = (m_run == -INFINITY ? 0.f : m_run) * scale_log2;
    float rs = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float p = fast_exp2(fmaf(sc[rr], scale_log2, -mb));
      sc[rr] = p;
      rs += p;
    }
    l_run = l_run * alpha + rs;

    u32x4 pb[2];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int r0 = 8 * mm;
      pb[mm] = u32x4{pack_bf16x2(sc[r0 + 0], sc[r0 + 1]), pack_bf16x2(sc[r0 + 2], sc[r0 + 3]),
                     pack_bf16x2(sc[r0 + 4], sc[r0 + 5]), pack_bf16x2(sc[r0 + 6], sc[r0 + 7])};
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = 32 * db + 16 * (tr_g & 1) + 4 * tr_t;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int row0 = 16 * mm + 4 * h + tr_j;
        const bf16x8 a = lds_read_tr16_pair(vls + row0 * C::VROW + col,
                                            vls + (row0 + 8) * C::VROW + col);
        oacc[db] = mfma32x32x16(a, pb[mm], oacc[db]);
      }
    }
    wave_lds_sync();  // this block's LDS reads precede the next block's writes
  }

  // merge the 4 waves' (m, l, Oᵀ) into one locally normalised partial for the split
  const float l_tot = pair32_sum(l_run);
  __syncthreads();
  float* ocb = (float*)smem;                // [NW][32][OROW] unnormalised Oᵀ rows
  float* mlb = ocb + C::NW * 32 * C::OROW;  // [NW][32][3]: exact max, reference max, sum
                                            // (score units; the sum is against the reference)
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *(f32x4*)(ocb + (wave * 32 + l32) * C::OROW + 32 * db + 8 * g4 + 4 * h) =
          f32x4{oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2],
                oacc[db][4 * g4 + 3]};
  if (h == 0) {
    mlb[(wave * 32 + l32) * 3 + 0] = m_true;
    mlb[(wave * 32 + l32) * 3 + 1] = m_run;
    mlb[(wave * 32 + l32) * 3 + 2] = l_tot;
  }
  __syncthreads();

  constexpr int DE = D / 8;  // head-dim elements per thread in the merge
  const int qr = tid >> 3, ch = tid & 7;
  const int rr = rg * 32 + qr;
  if (rr < R) {
    const int g2 = rr / Nq, qi2 = rr - g2 * Nq;
    const int hq2 = hkv * G + g2;
    // M = exact max of the split; each wave's sum and accumulator are re-expressed against it
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < C::NW; ++w)
      if (mlb[(w * 32 + qr) * 3 + 2] > 0.f) M = fmaxf(M, mlb[(w * 32 + qr) * 3]);
    float ew[C::NW];
    float Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) {
      const float lw = mlb[(w * 32 + qr) * 3 + 2];
      ew[w] = lw > 0.f ? fast_exp2((mlb[(w * 32 + qr) * 3 + 1] - M) * scale_log2) : 0.f;
      Lsum += ew[w] * lw;
    }
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    const size_t slot = (((size_t)b * Hq + hq2) * Nq + qi2) * S + s;
    float* dst = wsO + slot * D + ch * DE;
#pragma unroll
    for (int e = 0; e < DE; e += 4) {
      f32x4 o = f32x4{};
#pragma unroll
      for (int w = 0; w < C::NW; ++w)
        o += ew[w] * *(const f32x4*)(ocb + (w * 32 + qr) * C::OROW + ch * DE + e);
      *(f32x4*)(dst + e) = o * inv;
    }
    if (ch == 0) {
      wsML[slot * 2 + 0] = Lsum > 0.f ? M * scale : -INFINITY;
      wsML[slot * 2 + 1] = Lsum;
    }
  }
}

// max / sum over the 64 lanes of a wave (every lane gets the result)
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// One wave per output row (batch, query head, position).  Lane s reads the metadata of split s
// (64 splits per pass), so all metadata loads are in flight together; the weights
// w_s = l_s exp(m_s - M) are then broadcast lane by lane while the partial rows stream in.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ wsO,
                                                           const float* __restrict__ wsML,
                                                           uint16_t* __restrict__ O,
                                                           float* __restrict__ LSE, int rows,
                                                           int S) {
  constexpr int E = D / 64;  // head-dim elements per lane
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  if (row >= rows) return;
  const f32x2* ml = (const f32x2*)(wsML + (size_t)row * S * 2);
  float M = -INFINITY;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const f32x2 v = (s0 + lane < S) ? ml[s0 + lane] : f32x2{-INFINITY, 0.f};
    M = fmaxf(M, v[1] > 0.f ? v[0] : -INFINITY);
  }
  M = wave_max(M);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float W = 0.f;
  const float* src = wsO + (size_t)row * S * D + lane * E;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int n = min(64, S - s0);
    const f32x2 v = (lane < n) ? ml[s0 + lane] : f32x2{-INFINITY, 0.f};
    const float w = v[1] > 0.f ? v[1] * fast_exp2((v[0] - M) * kLog2e) : 0.f;
    W += w;
#pragma unroll 8
    for (int j = 0; j < n; ++j) {
      const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                     __builtin_bit_cast(int, w), j));
      const float* p = src + (size_t)(s0 + j) * D;
      if constexpr (E == 2) {
        const f32x2 o = *(const f32x2*)p;
        acc[0] = fmaf(wj, o[0], acc[0]);
        acc[1] = fmaf(wj, o[1], acc[1]);
      } else {
        acc[0] = fmaf(wj, p[0], acc[0]);
      }
    }
  }
  W = wave_sum(W);
  const float inv = W > 0.f ? 1.f / W : 0.f;
  uint16_t* dst = O + (size_t)row * D + lane * E;
  if constexpr (E == 2) {
    *(uint32_t*)dst = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
    dst[0] = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xffffu);
  }
  if (LSE != nullptr && lane == 0) LSE[row] = W > 0.f ? M + logf(W) : -INFINITY;
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* out, float* lse,
                  float* ws_o, float* ws_ml, const AttnShape& sh, float scale, int S,
                  hipStream_t stream) {
  using C = DecCfg<D>;
  const int L = (sh.Nk + S - 1) / S;
  const int R = (sh.Hq / sh.Hkv) * sh.Nq;
  const int nrg = (R + 31) / 32;
  const long long blocks = (long long)sh.B * sh.Hkv * nrg * S;
  const long long rows = (long long)sh.B * sh.Hq * sh.Nq;
  if (blocks > 0x7fffffffLL || rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(C::NT), 0,
                     stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, ws_o,
                     ws_ml, sh.Hq, sh.Hkv, sh.Nq, sh.Nk, S, L, nrg, scale, scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)rows), dim3(64), 0,
                     stream, (const float*)ws_o, (const float*)ws_ml, (uint16_t*)out, lse,
                     (int)rows, S);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_splitkv(const void* q, const void* k, const void* v, void* out,
                                 float* lse, float* ws_o, float* ws_ml, const AttnShape& s,
                                 float scale, bool causal, int n_splits, hipStream_t stream) {
  if (s.d == 128)
    return causal ? launch<128, true>(q, k, v, out, lse, ws_o, ws_ml, s, scale, n_splits, stream)
                  : launch<128, false>(q, k, v, out, lse, ws_o, ws_ml, s, scale, n_splits,
                                       stream);
  return causal ? launch<64, true>(q, k, v, out, lse, ws_o, ws_ml, s, scale, n_splits, stream)
                : launch<64, false>(q, k, v, out, lse, ws_o, ws_ml, s, scale, n_splits, stream);
}

}  // namespace fa
