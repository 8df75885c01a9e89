// Fused attention forward (prefill) for gfx950, bf16 in/out, fp32 accumulation.
//
// Method: the FlashAttention-2 forward ("FlashAttention-2: Faster Attention with Better
// Parallelism and Work Partitioning", section "방법론 / 알고리즘 개요"): for a block of query rows,
// loop over K/V blocks keeping a running row max m and row sum l, rescale the output accumulator
// by exp(m_old - m_new), and divide by l once at the end.  Blocks above the causal diagonal are
// never visited and only blocks straddling it are masked (section "인과적 마스킹 최적화").  The grid
// runs over batch x heads x query blocks (section "개선 2"), and each wavefront owns its own query
// rows so no cross-wave reduction is needed (section "개선 3").  The score matrix lives only in
// registers, never in memory.
//
// gfx950 mapping (one workgroup = 4 wavefronts = 128 query rows; K/V blocks of 64 keys):
//   * Each wave computes Sᵀ = K·Qᵀ (keys x its 32 queries) with v_mfma_f32_32x32x16_bf16: A = K
//     from LDS (one 16-byte read per lane), B = Qᵀ held in registers for the whole loop.  In the
//     accumulator layout lane l holds 32 key scores of query l%32, so the row max/sum are in-lane
//     plus one permlane32 swap with lane l^32.
//   * Oᵀ += Vᵀ·Pᵀ on the same MFMA: Pᵀ is the B operand straight from the score registers (packed
//     to bf16); the matching key order of Vᵀ comes from the transposing LDS read ds_read_b64_tr_b16,
//     so V stays row-major in LDS.  Every Oᵀ accumulator of a lane belongs to its own query, so the
//     rescale by exp2((m_old - m_new)·scale·log2e) is a per-lane scalar multiply, and it is only
//     done when some row's max grew by more than 2^8 (lazy rescaling; O and l keep one reference).
//   * K/V blocks go from HBM straight into LDS (buffer_load ... lds, 16 bytes per lane, no
//     register staging), double buffered: the next block's loads are issued right after the
//     barrier that publishes the current one.  Rows past the end of K/V read as zero through the
//     buffer range check.  Rows are stored unpadded with their 16-byte chunks XOR-swizzled, K and
//     V each with the swizzle that makes its read pattern conflict-free on the 64 LDS banks.
//   * Workgroups are ordered heaviest-first under the causal mask, and all query blocks of one
//     (batch, head) are kept on one XCD so their shared K/V stays in that XCD's L2.
#include "fa_device.h"
#include "fa_kernels.h"

#include <math.h>

namespace fa {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int BR = 128;                     // query rows per workgroup
  static constexpr int BC = 64;                      // keys per K/V block
  static constexpr int NT = 256;                     // threads per workgroup (4 waves)
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int TILE = BC * D;                // bf16 elements per K or V block
  static constexpr int STAGE = 2 * TILE;             // one K block + one V block
  static constexpr int RPL = 64 / CPR;               // rows covered by one wave-wide 1 KB load
  static constexpr int LPW = BC / RPL / 4;           // 1 KB loads per wave per tensor per block
  static_assert(BC % (4 * RPL) == 0, "staging must divide evenly");
};

// Physical 16-byte chunk of logical chunk c in row `row` (XOR swizzle, an involution).
// K rows are read 16 lanes = 16 consecutive rows at one logical chunk per LDS cycle; V rows by
// transposing reads, 32 lanes = 4 consecutive rows x 4 consecutive chunks per cycle.  Each
// swizzle maps those sets onto 16 distinct bank quads.
template <int D>
__device__ __forceinline__ int k_chunk(int row, int c) {
  return D == 128 ? (c ^ (row & 15)) : (c ^ ((row >> 1) & 7));
}
template <int D>
__device__ __forceinline__ int v_chunk(int row, int c) {
  return D == 128 ? (c ^ ((row & 3) << 2)) : (c ^ (((row >> 1) & 1) << 2));
}

// Block index -> (batch*head, query block).  Heaviest query blocks first (the last ones under a
// causal mask); when B*H is a multiple of 8 the blocks of a head go to one XCD (the dispatcher
// places block n on XCD n % 8).  When the whole grid fits in one round of workgroups (two per
// CU), the second half of an XCD's slots takes the blocks light-first, so that the two
// workgroups a CU receives carry about the same total causal work.
__device__ __forceinline__ void map_block(int n, int BH, int nqt, int& bh, int& qt) {
  if ((BH & 7) == 0) {
    const int xcd = n & 7, slot = n >> 3, hx = BH >> 3;
    const int S = hx * nqt;  // this XCD's workgroups, ranked by decreasing work
    int unit = slot;
    if (BH * nqt <= 512) {
      const int half = (S + 1) / 2;
      unit = slot < half ? slot : S - 1 - (slot - half);
    }
    bh = xcd * hx + unit % hx;
    qt = nqt - 1 - unit / hx;
  } else {
    bh = n % BH;
    qt = nqt - 1 - n / BH;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq,
    int Hkv, int Nq, int Nk, int nqt, float scale, float scale_log2) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int BH = gridDim.x / nqt;
  int bh, qt;
  map_block(blockIdx.x, BH, nqt, bh, qt);
  const int b = bh / Hq, hq = bh - b * Hq;
  const int hkv = hq / (Hq / Hkv);
  const int off = Nk - Nq;  // causal: key j visible to query i iff j <= i + off
  const int q_tile0 = qt * C::BR;
  const int qw0 = q_tile0 + wave * 32;  // first query row of this wave
  const int my_q = qw0 + l32;

  const uint32_t kv_bytes = (uint32_t)Nk * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + (size_t)(b * Hkv + hkv) * Nk * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + (size_t)(b * Hkv + hkv) * Nk * D, kv_bytes);

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(Nq - 1, q_tile0 + C::BR - 1) + off + 1);
  const int n_tiles = kv_end > 0 ? (kv_end + C::BC - 1) / C::BC : 0;

  // Qᵀ as the MFMA B operand: lane holds query my_q, head-dim slots 16c + 8h .. +7.
  u32x4 qf[D / 16];
  {
    const uint16_t* qrow = Q + ((size_t)bh * Nq + my_q) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qf[c] = (my_q < Nq) ? *(const u32x4*)(qrow + 16 * c + 8 * h) : u32x4{0u, 0u, 0u, 0u};
  }

  // This lane's slot in the wave's 1 KB direct loads: row within the load, physical chunk.
  const int ld_row = lane / C::CPR, ld_chunk = lane % C::CPR;
  auto issue_loads = [&](int t, int buf) {
    uint16_t* kbase = smem + buf * C::STAGE;
    uint16_t* vbase = kbase + C::TILE;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int blk = wave * C::LPW + i;  // which 1 KB piece of the block
      const int row = blk * C::RPL + ld_row;
      const uint32_t rowoff = (uint32_t)(t * C::BC + row) * (D * 2);
      load_lds_16(krs, kbase + blk * 512, rowoff + 16u * k_chunk<D>(row, ld_chunk));
      load_lds_16(vrs, vbase + blk * 512, rowoff + 16u * v_chunk<D>(row, ld_chunk));
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // transposing-read coordinates of this lane (see the layout note in fa_device.h)
  const int tr_g = lane >> 4, tr_j = (lane & 15) >> 2, tr_t = lane & 3;

  if (n_tiles > 0) issue_loads(0, 0);

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    wait_vmem();       // this wave's share of block t has landed in LDS
    __syncthreads();   // ... and everyone's; everyone is also done reading the other buffer
    if (t + 1 < n_tiles) issue_loads(t + 1, buf ^ 1);
    const uint16_t* ks = smem + buf * C::STAGE;
    const uint16_t* vs = ks + C::TILE;
    const int k0 = t * C::BC;
    const bool active = (qw0 < Nq) && (!CAUSAL || k0 <= qw0 + 31 + off);
    if (active) {
      // Sᵀ = K·Qᵀ for two 32-key halves of the block; all K operands are read up front
      u32x4 kop[2][D / 16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + l32;
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
          kop[kb][c] = *(const u32x4*)(ks + row * D + 8 * k_chunk<D>(row, 2 * c + h));
      }
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int c = 0; c < D / 16; ++c) s[kb] = mfma32x32x16(kop[kb][c], qf[c], s[kb]);
      }
      // mask keys past Nk and, on diagonal blocks, keys after this row's last visible key
      const bool need_mask = (k0 + C::BC > Nk) || (CAUSAL && (k0 + C::BC - 1 > qw0 + off));
      if (need_mask) {
        const int lim = CAUSAL ? min(Nk - 1, my_q + off) : Nk - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key > lim) s[kb][r] = -INFINITY;
          }
      }
      // online softmax (per lane = per query): block max, lazily moved reference max, rescale,
      // exponentiate, running sum
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = pair32_max(mx);
      const bool grow = (mx - m_run) * scale_log2 > kLazyLog2;  // false while both are -inf
      const float m_next = grow ? mx : m_run;
      const float alpha = grow ? fast_exp2((m_run - m_next) * scale_log2) : 1.f;
      if (wave_any(grow && m_run != -INFINITY)) {  // an already-started row moves its max
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      }
      m_run = m_next;
      const float mb = (m_run == -INFINITY ? 0.f : m_run) * scale_log2;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[kb][r], scale_log2, -mb));
          s[kb][r] = p;
          rs += p;
        }
      l_run = l_run * alpha + rs;  // lane-half partial; the partner half is added at the end

      // Pᵀ as B operands: block kb, 16-key group mm uses score registers 8mm .. 8mm+7
      u32x4 pb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const int r0 = 8 * mm;
          pb[2 * kb + mm] = u32x4{pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]),
                                  pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]),
                                  pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]),
                                  pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7])};
        }
      // Oᵀ += Vᵀ·Pᵀ.  Operand slot 8h + 4c + j of group (kb, mm) holds key
      // 32kb + 16mm + 8c + 4h + j, matching the score register order above.
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int chunk = 4 * db + 2 * (tr_g & 1) + (tr_t >> 1);
        const int within = 4 * (tr_t & 1);
        bf16x8 vop[4];
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
          const int r0 = 16 * m4 + 4 * h + tr_j, r1 = r0 + 8;
          vop[m4] = lds_read_tr16_pair(vs + r0 * D + 8 * v_chunk<D>(r0, chunk) + within,
                                       vs + r1 * D + 8 * v_chunk<D>(r1, chunk) + within);
        }
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) oacc[db] = mfma32x32x16(vop[m4], pb[m4], oacc[db]);
      }
    }
  }

  // epilogue: one 1/l per row, bf16 output, natural-log logsumexp
  const float l_tot = pair32_sum(l_run);
  if (my_q < Nq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = O + ((size_t)bh * Nq + my_q) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const u32x2 w = {pack_bf16x2(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv),
                         pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
        *(u32x2*)(orow + 32 * db + 8 * g4 + 4 * h) = w;
      }
    if (LSE != nullptr && h == 0)
      LSE[(size_t)bh * Nq + my_q] = l_tot > 0.f ? m_run * scale + logf(l_tot) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* out, float* lse,
                  const AttnShape& s, float scale, hipStream_t stream) {
  using C = FwdCfg<D>;
  const int nqt = (s.Nq + C::BR - 1) / C::BR;
  const long long blocks = (long long)s.B * s.Hq * nqt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(C::NT), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)out,
                     lse, s.Hq, s.Hkv, s.Nq, s.Nk, nqt, scale, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                           const AttnShape& s, float scale, bool causal, hipStream_t stream) {
  if (s.d == 128)
    return causal ? launch<128, true>(q, k, v, out, lse, s, scale, stream)
                  : launch<128, false>(q, k, v, out, lse, s, scale, stream);
  return causal ? launch<64, true>(q, k, v, out, lse, s, scale, stream)
                : launch<64, false>(q, k, v, out, lse, s, scale, stream);
}

}  // namespace fa
