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
//     so V stays row-major in LDS.  Every Oᵀ accumulator of a lane belongs to its own query, so a
//     rescale is a per-lane scalar multiply.
//   * Lazy rescaling: exponents are taken against a reference max that only moves when a block
//     holds a score more than 2^8 above it (in exp2 units), so probabilities stay below 2^8 and O
//     and l, which share the reference, are rarely rescaled.  The common case needs no block max:
//     the max of the exponent arguments is checked after the fact, and the rare block that
//     exceeds the bound is redone against its own max (scores recomputed from global K).
//   * Software pipelining: in steady state a step exponentiates block t while issuing block
//     t+1's QK products, instruction by instruction (scheduling fences keep the order), and then
//     issues block t's PV products 16 keys at a time while the next 16 keys are exponentiated.
//     The matrix cores therefore run while the transcendental and VALU work issues.  The PV part
//     is issued at raised wave priority, so the SIMD's other wave, in its vector-heavy QK part,
//     fills the gaps between these products.  Blocks that need a mask (the causal diagonal, a
//     ragged end) run an unpipelined step instead.
//   * K/V blocks go from HBM straight into LDS (buffer_load ... lds, 16 bytes per lane, no
//     register staging).  K runs one block ahead of V: at the start of step t, K[t+1] and V[t]
//     are in LDS and K[t+2], V[t+1] are requested, so two buffers each suffice; every buffer is
//     its own LDS variable so the compiler can tell the in-flight copies from the reads.  Rows
//     past the end of K/V read as zero through the buffer range check.  Rows are stored unpadded
//     with their 16-byte chunks XOR-swizzled, K and V each with the swizzle that makes its read
//     pattern conflict-free on the 64 LDS banks.
//   * Workgroups are ordered heaviest-first under the causal mask, and all query blocks of one
//     (batch, head) are kept on one XCD so their shared K/V stays in that XCD's L2.  When the grid
//     spans several rounds of workgroups, a workgroup instead takes query blocks nqt-1-i and i of
//     one head in turn (equal causal work per workgroup), heads in order within each XCD, so the
//     workgroups of a head start together and stream its K/V through L2 side by side.
#include "fa_device.h"
#include "fa_kernels.h"

#include <math.h>

#include <type_traits>

namespace fa {
namespace {

constexpr long long kPairedMinGrid = 512;  // MI355X: 256 CUs x 2 workgroups

template <int D>
struct FwdCfg {
  static constexpr int BR = 128;                     // query rows per workgroup
  static constexpr int BC = 64;                      // keys per K/V block
  static constexpr int NT = 256;                     // threads per workgroup (4 waves)
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int TILE = BC * D;                // bf16 elements per K or V block
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

// One query block (bh, qt) of the forward: the whole FlashAttention-2 loop over its K/V blocks.
template <int D, bool CAUSAL, bool BIAS>
__device__ __forceinline__ void fwd_tile(
    int bh, int qt, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    const int* __restrict__ seqlens, const uint16_t* __restrict__ bias, int bias_b, int bias_h,
    int Hq, int Hkv, int Nq, int Nk_cap, float scale, float scale_log2) {
  using C = FwdCfg<D>;
  constexpr int NC = D / 16;  // 16-element head-dim slices per QK product
  __shared__ __attribute__((aligned(1024))) uint16_t kl0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t kl1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vl0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vl1[C::TILE];
  // bias: each wave's 32 rows x BC keys, one buffer per wave (16 KB in all, so that two
  // workgroups still fit a CU's 160 KB)
  __shared__ __attribute__((aligned(1024))) uint16_t bl[BIAS ? 4 * 32 * C::BC : 8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int b = bh / Hq, hq = bh - b * Hq;
  const int hkv = hq / (Hq / Hkv);
  // keys of this batch element: all Nk_cap rows of K/V, or the first seqlens[b] (clamped)
  const int Nk = seqlens ? min(max(seqlens[b], 0), Nk_cap) : Nk_cap;
  const int off = Nk - Nq;  // causal: key j visible to query i iff j <= i + off
  const int q_tile0 = qt * C::BR;
  const int qw0 = q_tile0 + wave * 32;  // first query row of this wave
  const int my_q = qw0 + l32;

  const uint32_t kv_bytes = (uint32_t)Nk * D * 2;
  const uint16_t* kg = K + (size_t)(b * Hkv + hkv) * Nk_cap * D;
  const uint16_t* vg = V + (size_t)(b * Hkv + hkv) * Nk_cap * D;

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(Nq - 1, q_tile0 + C::BR - 1) + off + 1);
  const int n_tiles = kv_end > 0 ? (kv_end + C::BC - 1) / C::BC : 0;

  u32x4 qf[NC];
  {
    const uint16_t* qrow = Q + ((size_t)bh * Nq + my_q) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[c] = (my_q < Nq) ? *(const u32x4*)(qrow + 16 * c + 8 * h) : u32x4{0u, 0u, 0u, 0u};
  }

  // Direct loads: the buffer resource of block t starts at that block and covers the rest of K
  // (or V), so a lane's offset is the same for every block; rows past Nk read as zero.  Load i
  // of a wave fills rows (4i + wave)·RPL .. +RPL-1, which keeps each lane's swizzled chunk the
  // same for every i: the i-dependent part is a plain byte offset, passed as the scalar offset.
  const int ld_row = lane / C::CPR, ld_chunk = lane % C::CPR;
  const int row0 = wave * C::RPL + ld_row;
  const uint32_t koff = (uint32_t)row0 * (D * 2) + 16u * k_chunk<D>(row0, ld_chunk);
  const uint32_t voff = (uint32_t)row0 * (D * 2) + 16u * v_chunk<D>(row0, ld_chunk);
  auto issue = [&](const uint16_t* g, int t, uint16_t* dst, uint32_t lane_off) {
    // a block at or past the end gets an empty resource: every lane reads zero
    const uint32_t skip = (uint32_t)min(t * C::BC, Nk) * (D * 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(g + (size_t)skip / 2, kv_bytes - skip);
#pragma unroll
    for (int i = 0; i < C::LPW; ++i)
      load_lds_16(rs, dst + (4 * i + wave) * 512, lane_off, (uint32_t)i * (4 * C::RPL * D * 2));
  };
  auto issue_k = [&](int t, uint16_t* dst) { issue(kg, t, dst, koff); };
  auto issue_v = [&](int t, uint16_t* dst) { issue(vg, t, dst, voff); };

  // LDS read addresses.  Rows start on 256-byte (D = 128) or 128-byte (D = 64) boundaries and
  // every swizzle XORs the logical chunk index with a function of the row, so the address of
  // logical chunk c is this lane's address of chunk 0 XOR (16 c): one VALU op per read.
  const uint32_t k_lane = (uint32_t)(l32 * D + 8 * k_chunk<D>(l32, h)) * 2;
  const int tr_g = lane >> 4, tr_j = (lane & 15) >> 2, tr_t = lane & 3;
  const int v_r0 = 4 * h + tr_j;
  const uint32_t v_lane =
      (uint32_t)(v_r0 * D + 8 * v_chunk<D>(v_r0, 2 * (tr_g & 1) + (tr_t >> 1)) + 4 * (tr_t & 1)) * 2;
  // byte address of K operand (kb, c) / V operand base for head-dim block db, within a buffer
  auto k_addr = [&](const uint16_t* buf, int c) {
    return (const u32x4*)((const char*)buf + (k_lane ^ (32u * c)));
  };
  auto v_addr = [&](const uint16_t* buf, int db) {
    return (const uint16_t*)((const char*)buf + (v_lane ^ (64u * db)));
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Additive bias (bf16 [bias_b, bias_h, Nq, Nk_cap], batch and head dims broadcast when 1), in
  // score units (bias / scale).  A block's bias is the starting value of its score accumulators.
  // Each wave copies its own 32 rows x BC keys of bias into its LDS slice (four 1 KB copies of
  // eight 128-byte rows, coalesced) through a resource covering its rows (rows past Nq read
  // zero); the copy of block x+1 is requested once block x has been read out, and as a wave only
  // reads its own slice no barrier is involved.  Slot p of row 8i+j holds 16-byte chunk
  // p ^ f(i, j), f = (j >> 1) | ((i & 1) << 2): the 8-byte reads of one chunk by the 32 rows then
  // fall on distinct bank pairs within each half of the 64 banks.  The rarely taken path that
  // recomputes a block reads its bias from global memory instead.
  const size_t b_slice = ((size_t)(bias_b == 1 ? 0 : b) * bias_h + (bias_h == 1 ? 0 : hq)) * Nq;
  const __amdgpu_buffer_rsrc_t brs =
      make_rsrc(BIAS ? bias + (b_slice + (size_t)min(qw0, Nq)) * Nk_cap : nullptr,
                BIAS ? (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(32, Nq - qw0)) * Nk_cap * 2)
                     : 0u);
  const float inv_scale = 1.f / scale;
  const float inv_scale_log2 = 1.f / scale_log2;
  uint16_t* const bw = bl + (BIAS ? wave * 32 * C::BC : 0);
  const int bj = lane >> 3, bp = lane & 7;
  const uint32_t b_row = (uint32_t)bj * Nk_cap * 2, b_cw = (uint32_t)(bp ^ (bj >> 1)) << 4;
  auto issue_bias = [&](int t) {
    if constexpr (BIAS) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        load_lds_16(brs, bw + i * 8 * C::BC, b_row + (b_cw ^ ((i & 1) << 6)),
                    (uint32_t)(8 * i) * Nk_cap * 2 + (uint32_t)t * (C::BC * 2));
    }
  };
  // this lane's 8-byte read of logical chunk c (keys 8c .. 8c+7, half h) is b_rd ^ (16 c)
  const uint32_t b_rd = (uint32_t)l32 * (C::BC * 2) +
                        ((uint32_t)(((l32 & 7) >> 1) | (((l32 >> 3) & 1) << 2)) << 4) + 8u * h;
  auto bias_val = [&](uint32_t w, int odd) {
    return __uint_as_float(odd ? (w & 0xffff0000u) : (w << 16)) * inv_scale;
  };
  // zero, or the bias of the block whose scores come next (from this wave's LDS slice)
  auto init_scores = [&](f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (BIAS) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 w = *(const u32x2*)((const char*)bw + (b_rd ^ (uint32_t)((4 * kb + g) << 4)));
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kb][4 * g + e] = bias_val(w[e >> 1], e & 1);
        }
      } else {
        s[kb] = f32x16{};
      }
    }
  };
  // the same values of block t straight from global memory (eight 8-byte loads per lane)
  const uint32_t b_lane = ((uint32_t)l32 * Nk_cap + 4u * h) * 2u;
  auto add_bias_global = [&](f32x16 (&s)[2], int t) {
    if constexpr (BIAS) {
      u32x2 w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                   brs, (int)(b_lane + (uint32_t)((32 * (i >> 2) + 8 * (i & 3)) * 2)),
                   t * C::BC * 2, 0));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] += bias_val(w[4 * kb + (r >> 2)][(r >> 1) & 1], r & 1);
    }
  };

  auto active = [&](int t) { return (qw0 < Nq) && (!CAUSAL || t * C::BC <= qw0 + 31 + off); };

  // keys past Nk and, on diagonal blocks, keys after this row's last visible key -> -inf
  auto mask = [&](int k0, f32x16 (&s)[2]) {
    const bool need = (k0 + C::BC > Nk) || (CAUSAL && (k0 + C::BC - 1 > qw0 + off));
    if (need) {
      const int lim = CAUSAL ? min(Nk - 1, my_q + off) : Nk - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key > lim) s[kb][r] = -INFINITY;
        }
    }
  };

  // Sᵀ = K·Qᵀ of one block from LDS, K operands read one slice ahead
  auto scores_lds = [&](const uint16_t* ks, f32x16 (&s)[2]) {
    u32x4 ka0 = *k_addr(ks, 0);
    u32x4 ka1 = *(k_addr(ks, 0) + 32 * D / 8);
    init_scores(s);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 kn0 = ka0, kn1 = ka1;
      if (c + 1 < NC) {
        kn0 = *k_addr(ks, c + 1);
        kn1 = *(k_addr(ks, c + 1) + 32 * D / 8);
      }
      s[0] = mfma32x32x16(ka0, qf[c], s[0]);
      s[1] = mfma32x32x16(ka1, qf[c], s[1]);
      __builtin_amdgcn_sched_barrier(0);
      ka0 = kn0;
      ka1 = kn1;
    }
  };

  // The same straight from global memory (the rarely taken path that redoes a block), two
  // operands at a time
  auto scores_global = [&](int k0, f32x16 (&s)[2]) {
    const int row0 = k0 + l32, row1 = row0 + 32;
    const uint16_t* kr0 = kg + (size_t)min(row0, Nk - 1) * D + 8 * h;
    const uint16_t* kr1 = kg + (size_t)min(row1, Nk - 1) * D + 8 * h;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const u32x4 a0 = row0 < Nk ? *(const u32x4*)(kr0 + 16 * c) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 a1 = row1 < Nk ? *(const u32x4*)(kr1 + 16 * c) : u32x4{0u, 0u, 0u, 0u};
      s[0] = mfma32x32x16(a0, qf[c], s[0]);
      s[1] = mfma32x32x16(a1, qf[c], s[1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // exponent arguments x = s·scale·log2e - mb of score pair (j, j+1), in place, and their max.
  // The running max takes one three-input max per pair (a chain of v_max3, 16 per block of 32
  // arguments; the compiler's own reduction of the same expression used 24 operations).
  auto arg_pair = [&](f32x16 (&s)[2], float& amax, float mb, int j) {
    const int kb = j >> 4, r = j & 15;
    const float x0 = fmaf(s[kb][r], scale_log2, -mb);
    const float x1 = fmaf(s[kb][r + 1], scale_log2, -mb);
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(amax) : "v"(amax), "v"(x0), "v"(x1));
    s[kb][r] = x0;
    s[kb][r + 1] = x1;
  };
  // probabilities 2^x of pair (j, j+1), in place, packed into P
  auto exp_pair = [&](f32x16 (&s)[2], u32x4 (&pb)[4], int j) {
    const int kb = j >> 4, r = j & 15;
    const float p0 = fast_exp2(s[kb][r]), p1 = fast_exp2(s[kb][r + 1]);
    s[kb][r] = p0;
    s[kb][r + 1] = p1;
    const uint32_t pk = pack_bf16x2(p0, p1);
    asm volatile("" ::"v"(pk));
    pb[j >> 3][(j >> 1) & 3] = pk;
  };

  // The block's exact max becomes the reference: rescale O and l, recompute the arguments and
  // group 0's probabilities (only for blocks that need no mask).
  auto redo_block = [&](f32x16 (&s)[2], u32x4 (&pb)[4], int k0, float& mb) {
    scores_global(k0, s);
    add_bias_global(s, k0 / C::BC);  // the LDS slice already holds the next block
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = pair32_max(mx);
    const float m_next = fmaxf(m_run, mx);
    const float alpha = m_next == -INFINITY ? 1.f : fast_exp2((m_run - m_next) * scale_log2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    l_run *= alpha;
    m_run = m_next;
    mb = (m_run == -INFINITY ? 0.f : m_run) * scale_log2;
    float amax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 32; j += 2) arg_pair(s, amax, mb, j);
#pragma unroll
    for (int j = 0; j < 8; j += 2) exp_pair(s, pb, j);
  };

  // The block's arguments exceed the bound by at most kShiftMax: move the reference up by the
  // block's own largest argument in registers.  Arguments not yet exponentiated drop by that
  // amount, the probabilities already taken (group 0) and O, l scale by 2^-shift; rows within
  // the bound keep their reference.  Group 0's probabilities are at most 2^kShiftMax, finite.
  auto shift_block = [&](f32x16 (&s)[2], u32x4 (&pb)[4], float bmax) {
    const float sh = bmax > kLazyLog2 ? bmax : 0.f;
    const float alpha = fast_exp2(-sh);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    l_run *= alpha;
    m_run += sh * inv_scale_log2;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j < 8) s[j >> 4][j & 15] *= alpha;
      else s[j >> 4][j & 15] -= sh;
    }
#pragma unroll
    for (int j = 0; j < 8; j += 2) pb[0][j >> 1] = pack_bf16x2(s[0][j], s[0][j + 1]);
  };

  f32x16 sA[2], sB[2];

  // Blocks [0, n_free) need no mask for any wave of the workgroup: every key is below Nk and,
  // under the causal mask, visible to the workgroup's first query row.
  int n_free = Nk / C::BC;
  if (CAUSAL) n_free = min(n_free, max(0, (q_tile0 + off + 1) / C::BC));
  n_free = min(n_free, n_tiles);

  // Steady-state step for an unmasked block t (scores in `s`): block t's exponentials are
  // interleaved instruction by instruction with the QK products of block t+1 (into `sn`), so
  // the transcendental and VALU work issues while the matrix cores run; then Oᵀ += Vᵀ·Pᵀ for
  // block t, interleaved with the row sums.  Buffers: K[t] and V[t] live in kl/vl[t % 2]; at
  // the start of step t, K[t+1] and V[t] have landed, and K[t+2] and V[t+1] are requested.
  auto step = [&](int t, auto bufc, f32x16 (&s)[2], f32x16 (&sn)[2]) {
    constexpr int BUF = decltype(bufc)::value;
    uint16_t* const k_next = BUF ? kl0 : kl1;   // block t+1's keys
    uint16_t* const k_free = BUF ? kl1 : kl0;   // block t's keys, no longer read
    uint16_t* const v_cur = BUF ? vl1 : vl0;    // block t's values
    uint16_t* const v_next = BUF ? vl0 : vl1;
    wait_vmem();       // this wave's loads of K[t+1] and V[t] have landed ...
    __syncthreads();   // ... and everyone's; K[t] and V[t-1] are free again
    if (t + 2 < n_tiles) issue_k(t + 2, k_free);
    if (t + 1 < n_tiles && t >= 1) issue_v(t + 1, v_next);  // V[1] came with the prologue
    if (qw0 >= Nq) return;
    // Block t+1's products are always issued (when t+1 does not exist or is inactive for this
    // wave, they read whatever the buffer holds and the result is never used).  Interleaved with
    // them: block t's exponent arguments and max, and at the end group 0's probabilities.
    float mb = m_run * scale_log2;
    float amax = -INFINITY;
    u32x4 pb[4];
    constexpr int NS = 2 * NC;            // products in this part
    constexpr int APS = 32 / NS;          // arguments per product
    constexpr int G0 = NS - 4;            // first product that also takes group 0's exponentials
    {
      u32x4 kr[3][2];
      kr[0][0] = *k_addr(k_next, 0);
      kr[0][1] = *(k_addr(k_next, 0) + 32 * D / 8);
      kr[1][0] = *k_addr(k_next, 1);
      kr[1][1] = *(k_addr(k_next, 1) + 32 * D / 8);
      init_scores(sn);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c + 2 < NC) {
          kr[(c + 2) % 3][0] = *k_addr(k_next, c + 2);
          kr[(c + 2) % 3][1] = *(k_addr(k_next, c + 2) + 32 * D / 8);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int slot = 2 * c + hh;
          sn[hh] = mfma32x32x16(kr[c % 3][hh], qf[c], sn[hh]);
#pragma unroll
          for (int j = slot * APS; j < (slot + 1) * APS; j += 2) arg_pair(s, amax, mb, j);
          if (slot >= G0) exp_pair(s, pb, 2 * (slot - G0));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // an argument above kLazyLog2: shift the reference in registers, or, when the jump is
    // larger than kShiftMax or there is no reference yet, redo the block against its max
    if (wave_any(!(amax <= kLazyLog2) || m_run == -INFINITY)) {
      const float bmax = pair32_max(amax);
      const bool fast = wave_all(bmax <= kShiftMax && m_run != -INFINITY);
      // (not an if / else: the two paths' register demands would then add up)
      shift_block(s, pb, fast ? bmax : 0.f);  // a no-op when the block is redone
      if (!fast) redo_block(s, pb, t * C::BC, mb);
    }
    if (t + 2 < n_tiles) issue_bias(t + 2);  // block t+1's bias has been read out

    // Oᵀ += Vᵀ·Pᵀ, 16-key group by group (group g is operand pb[g]); while group g's products
    // run, group g+1's exponentials and group g's row sums are done.  V operands of group g+1
    // are read while group g's products run.  The wave issues this part at raised priority: the
    // SIMD's other wave, in the vector-heavy first part of its own step, then fills the gaps
    // between these products instead of delaying them (measured 3-7% on multi-round grids).
    constexpr int NDB = D / 32;
    __builtin_amdgcn_s_setprio(1);
    float rs = 0.f;
    bf16x8 vop[2][NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      vop[0][db] = lds_read_tr16_pair(v_addr(v_cur, db), v_addr(v_cur, db) + 8 * D);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if (g + 1 < 4)
          vop[(g + 1) & 1][db] = lds_read_tr16_pair(v_addr(v_cur, db) + 16 * (g + 1) * D,
                                                    v_addr(v_cur, db) + (16 * (g + 1) + 8) * D);
        oacc[db] = mfma32x32x16(vop[g & 1][db], pb[g], oacc[db]);
        // group g+1's exponentials: 8 values over this group's NDB products
#pragma unroll
        for (int j = 8 * (g + 1) + db * 8 / NDB; j < 8 * (g + 1) + (db + 1) * 8 / NDB; j += 2)
          if (g + 1 < 4) exp_pair(s, pb, j);
        // group g's row sums
#pragma unroll
        for (int j = 8 * g + db * 8 / NDB; j < 8 * g + (db + 1) * 8 / NDB; ++j)
          rs += s[j >> 4][j & 15];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    l_run += rs;  // lane-half partial; the partner half is added at the end
  };

  // Step for a block that may need masking (diagonal or ragged end), done in order: mask,
  // exact block max and lazy rescale, exponentials, PV, then block t+1's scores.  Same buffers.
  auto step_tail = [&](int t, f32x16 (&s)[2]) {
    const int k0 = t * C::BC;
    uint16_t* const k_next = (t & 1) ? kl0 : kl1;
    uint16_t* const k_free = (t & 1) ? kl1 : kl0;
    const uint16_t* const v_cur = (t & 1) ? vl1 : vl0;
    uint16_t* const v_next = (t & 1) ? vl0 : vl1;
    wait_vmem();
    __syncthreads();
    if (t + 2 < n_tiles) issue_k(t + 2, k_free);
    if (t + 1 < n_tiles && t >= 1) issue_v(t + 1, v_next);  // V[1] came with the prologue
    if (!active(t)) return;
    mask(k0, s);
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = pair32_max(mx);
    const bool grow = (mx - m_run) * scale_log2 > kLazyLog2;  // false while both are -inf
    const float m_next = grow ? mx : m_run;
    const float alpha = grow ? fast_exp2((m_run - m_next) * scale_log2) : 1.f;
    if (wave_any(grow && m_run != -INFINITY)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    m_run = m_next;
    const float mb = (m_run == -INFINITY ? 0.f : m_run) * scale_log2;
    float rs = 0.f, amax = -INFINITY;
    u32x4 pb[4];
#pragma unroll
    for (int j = 0; j < 32; j += 2) arg_pair(s, amax, mb, j);
#pragma unroll
    for (int j = 0; j < 32; j += 2) exp_pair(s, pb, j);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) rs += s[kb][r];
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      bf16x8 vop[4];
#pragma unroll
      for (int m4 = 0; m4 < 4; ++m4)
        vop[m4] = lds_read_tr16_pair(v_addr(v_cur, db) + 16 * m4 * D,
                                     v_addr(v_cur, db) + (16 * m4 + 8) * D);
#pragma unroll
      for (int m4 = 0; m4 < 4; ++m4) oacc[db] = mfma32x32x16(vop[m4], pb[m4], oacc[db]);
    }
    if (t + 1 < n_tiles && active(t + 1)) scores_lds(k_next, s);
    if (t + 2 < n_tiles) issue_bias(t + 2);
  };

  // prologue: K[0], V[0], K[1], V[1] are requested together (all four buffers are free), the
  // wave waits for K[0] only, then block 0's scores; when block 0 is unmasked its exact max
  // becomes the first reference.  Loads complete in issue order, so "at most 3·LPW loads
  // outstanding" means K[0] (and the Q rows loaded before it) have landed.
  if (n_tiles > 0) {
    issue_bias(0);  // before K[0], so the wait below covers it
    issue_k(0, kl0);
    issue_v(0, vl0);
    issue_k(1, kl1);
    issue_v(1, vl1);
    constexpr int later = 3 * C::LPW;
    __builtin_amdgcn_s_waitcnt(0x0F70 | (later & 15) | ((later >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();  // every wave's share of K[0] is in LDS
    asm volatile("" ::: "memory");
    if (active(0)) {
      scores_lds(kl0, sA);
      if (n_free > 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sA[kb][r]);
        m_run = pair32_max(mx);
      }
    }
    if (n_tiles > 1) issue_bias(1);
  }
  int t = 0;
  for (; t + 1 < n_free; t += 2) {
    step(t, std::integral_constant<int, 0>{}, sA, sB);
    step(t + 1, std::integral_constant<int, 1>{}, sB, sA);
  }
  if (t < n_free) {
    step(t, std::integral_constant<int, 0>{}, sA, sB);
    ++t;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sA[kb] = sB[kb];
  }
  for (; t < n_tiles; ++t) step_tail(t, sA);

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

// Paired grids (several rounds of workgroups): workgroup n runs on XCD n % 8 and takes, among
// that XCD's heads in order, head slot / np's query blocks nqt-1-i and i (i = slot % np, np =
// ceil(nqt / 2)), one after the other.  Every workgroup then carries the same causal work, and the
// workgroups of one head start together, so they stream its K/V through the XCD's L2 at the same
// time.  Other grids take one query block per workgroup (map_block).
template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    const int* __restrict__ seqlens, const uint16_t* __restrict__ bias, int bias_b, int bias_h,
    int Hq, int Hkv, int Nq, int Nk_cap, int nqt, int BH, int paired, float scale,
    float scale_log2) {
  int bh, qt, qt2 = -1;
  if (paired) {
    const int np = (nqt + 1) / 2, hx = BH >> 3;
    const int slot = blockIdx.x >> 3;
    bh = (blockIdx.x & 7) * hx + slot / np;
    const int i = slot % np;
    qt = nqt - 1 - i;
    if (i != qt) qt2 = i;
  } else {
    map_block(blockIdx.x, BH, nqt, bh, qt);
  }
  fwd_tile<D, CAUSAL, BIAS>(bh, qt, Q, K, V, O, LSE, seqlens, bias, bias_b, bias_h, Hq, Hkv, Nq,
                            Nk_cap, scale, scale_log2);
  if (qt2 >= 0) {
    __syncthreads();  // every wave is done with the first block's LDS buffers
    fwd_tile<D, CAUSAL, BIAS>(bh, qt2, Q, K, V, O, LSE, seqlens, bias, bias_b, bias_h, Hq, Hkv,
                              Nq, Nk_cap, scale, scale_log2);
  }
}

template <int D, bool CAUSAL, bool BIAS>
hipError_t launch(const void* q, const void* k, const void* v, void* out, float* lse,
                  const int* seqlens, const void* bias, int bias_b, int bias_h,
                  const AttnShape& s, float scale, hipStream_t stream) {
  using C = FwdCfg<D>;
  const int nqt = (s.Nq + C::BR - 1) / C::BR;
  const long long blocks = (long long)s.B * s.Hq * nqt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int BH = s.B * s.Hq;
  // pair query blocks when even the paired grid fills every slot of the chip (256 CUs x 2)
  const long long pairs = (long long)BH * ((nqt + 1) / 2);
  const int paired = (BH % 8 == 0 && nqt > 1 && pairs >= kPairedMinGrid) ? 1 : 0;
  const unsigned grid = paired ? (unsigned)pairs : (unsigned)blocks;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, BIAS>), dim3(grid), dim3(C::NT), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)out,
                     lse, seqlens, (const uint16_t*)bias, bias_b, bias_h, s.Hq, s.Hkv, s.Nq,
                     s.Nk, nqt, BH, paired, scale, scale * kLog2e);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_b(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int* seqlens, const void* bias, int bias_b, int bias_h,
                    const AttnShape& s, float scale, hipStream_t stream) {
  return bias ? launch<D, CAUSAL, true>(q, k, v, out, lse, seqlens, bias, bias_b, bias_h, s, scale,
                                        stream)
              : launch<D, CAUSAL, false>(q, k, v, out, lse, seqlens, nullptr, 1, 1, s, scale,
                                         stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                           const int* seqlens, const void* bias, int bias_b, int bias_h,
                           const AttnShape& s, float scale, bool causal, hipStream_t stream) {
  if (s.d == 128)
    return causal ? launch_b<128, true>(q, k, v, out, lse, seqlens, bias, bias_b, bias_h, s,
                                        scale, stream)
                  : launch_b<128, false>(q, k, v, out, lse, seqlens, bias, bias_b, bias_h, s,
                                         scale, stream);
  return causal ? launch_b<64, true>(q, k, v, out, lse, seqlens, bias, bias_b, bias_h, s, scale,
                                     stream)
                : launch_b<64, false>(q, k, v, out, lse, seqlens, bias, bias_b, bias_h, s, scale,
                                      stream);
}

}  // namespace fa
