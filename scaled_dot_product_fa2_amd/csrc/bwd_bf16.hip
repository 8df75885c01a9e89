// Attention backward for gfx950, bf16 in/out, fp32 accumulation (head dims 64 and 128).
//
// Not on the pages (they give only the speedups of the backward pass).  The gradients of
// L = sum(dO * O) through O = softmax(scale * Q K^T + causal mask) V are, with P recomputed from
// the forward's logsumexp (P = exp(scale * S - LSE)):
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D_i = sum_d dO_id O_id,
//     dQ = scale * dS K,   dK = scale * dS^T Q,
// (D_i equals sum_k P_ik dP_ik, the softmax Jacobian's centring term, because O = P V).  Key and
// value heads shared by several query heads receive the sum over those heads.
//
// gfx950 mapping, two launches on one stream:
//   * bwd_dq_kernel: the forward's structure.  A workgroup owns 128 query rows (32 per wave, Q
//     and dO held in registers as the B operand); 64-key blocks of K and V stream HBM -> LDS.
//     It also computes each row's D from O and dO and writes the row terms -D and -LSE / scale
//     to the workspace; they start the dK/dV kernel's score accumulators, which therefore end as
//     dP - D and S - LSE / scale.
//     S^T = K Q^T and dP^T = V dO^T on v_mfma_f32_32x32x16_bf16 put one query per lane, so P and
//     dS are per-lane formulas with the row's LSE and D; dQ^T += K^T dS^T takes K^T from the
//     transposing LDS read and dS^T straight from the registers.
//   * bwd_dkdv_kernel: the transpose of that.  A workgroup owns 128 keys (32 per wave pair);
//     64-row blocks of Q and dO (and their row terms) stream through LDS, over every query head that
//     shares the K/V head.  S = Q K^T and dP = dO V^T put one key per lane; eight waves share each
//     block: four compute S, P and dV^T += dO^T P, four dP and, with P passed through LDS one step
//     later, dS and dK^T += Q^T dS, so each wave runs two products and holds one accumulator set
//     (two waves per SIMD).  dK and dV need no atomics and are deterministic.
//   The LDS tiles use one XOR swizzle, chunk c of row r at c ^ ((r & 3) << 2 | (r >> 2) & 3),
//   under which both access patterns are conflict-free: 16 consecutive rows at one chunk (the
//   row-wise operand reads) and 4 consecutive rows x 4 chunks (the transposing reads).
//   In both kernels the first products' operands are read from LDS a few slices ahead into a
//   register ring, fenced so that the compiler keeps the distance.
#include "fa_device.h"
#include "fa_kernels.h"

#include <math.h>

#include <type_traits>
namespace fa {
namespace {

constexpr int BT = 64;  // rows per streamed block (keys in dq, queries in dkdv)

// Tile geometry for head dimension D (64 or 128).  A block of BT rows is stored unpadded, rows of
// 2D bytes, with 16-byte chunks XOR-swizzled so that both LDS read patterns are conflict-free on
// the 64 banks:
//   D = 128 (256-byte rows): chunk c of row r at c ^ ((r & 3) << 2 | (r >> 2) & 3);
//   D = 64 (128-byte rows, two rows per 256-byte line of banks): c ^ rev3((r >> 1) & 7), rev3
//   reversing three bits.
// The row-wise operand reads take 16 consecutive rows at one chunk; the transposing reads take
// 4 consecutive rows x 4 chunks per 32 lanes.  Row r + 8 differs from row r by chunk bit 1
// (D = 128) or bit 0 (D = 64): the second read of a transposing pair XORs that in (R8 bytes).
template <int D>
struct Geo {
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  static constexpr int RB = 2 * D;                      // bytes per row
  static constexpr int TILE = BT * D;                   // bf16 elements of one block
  static constexpr int NCB = D / 16;                    // 16-dim slices per product
  static constexpr int NDB = D / 32;                    // 32-dim output tiles
  static constexpr int CPR = D / 8;                     // 16-byte chunks per row
  static constexpr int RPL = 1024 / RB;                 // rows per 1 KB copy
  static constexpr int LPW = BT / RPL / 4;              // 1 KB copies per wave per block
  static constexpr uint32_t R8 = D == 128 ? 32u : 16u;  // byte XOR from row r to row r + 8
  __device__ static __forceinline__ int swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    const int x = (row >> 1) & 7;
    return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
  }
};

// The lane's byte offsets inside a swizzled [BT][D] tile.
//   row_base: row-wise A operand (rows x dims): lane (l32, h) reads row l32, dims 16c + 8h .. +7
//     (logical chunk 2c + h); the address of slice c is row_base ^ (32 c); rows 32..63 are
//     + 32 RB bytes.
//   tr_base: transposing A operand (dims x rows) for the key/query order of the C layout; the
//     operand of dim block db over rows R + (0..7, 8..15) is read at
//     ((tr_base ^ (64 db)) + R RB) and ((tr_base ^ (64 db) ^ R8) + (R + 8) RB), R = 16 g.
struct TileLanes {
  uint32_t row_base, tr_base;
};
template <int D>
__device__ __forceinline__ TileLanes tile_lanes(int lane) {
  using G = Geo<D>;
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_g = lane >> 4, tr_j = (lane & 15) >> 2, tr_t = lane & 3;
  const int r0 = 4 * h + tr_j, cl = 2 * (tr_g & 1) + (tr_t >> 1);
  TileLanes t;
  t.row_base = (uint32_t)(l32 * G::RB + 16 * (h ^ G::swz(l32)));
  t.tr_base = (uint32_t)(r0 * G::RB + 16 * (cl ^ G::swz(r0)) + 8 * (tr_t & 1));
  return t;
}
template <int D>
__device__ __forceinline__ u32x4 read_row(const uint16_t* tile, uint32_t row_base, int half, int c) {
  return *(const u32x4*)((const char*)tile + half * 32 * Geo<D>::RB + (row_base ^ (32u * c)));
}
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const uint16_t* tile, uint32_t tr_base, int R, int db) {
  using G = Geo<D>;
  const char* b = (const char*)tile;
  const uint32_t a = tr_base ^ (64u * db);
  return lds_read_tr16_pair((const uint16_t*)(b + a + R * G::RB),
                            (const uint16_t*)(b + (a ^ G::R8) + (R + 8) * G::RB));
}

// Copy rows [r0, r0 + BT) of a [n_rows][D] bf16 matrix into a swizzled LDS tile: 4 waves x LPW
// loads of 1 KB (RPL rows each); rows at or past n_rows read as zero.  Load i of wave w fills
// rows RPL (4 i + w) .. +RPL-1, so the swizzled chunk of a lane does not depend on i.
template <int D>
__device__ __forceinline__ void copy_tile(const uint16_t* g, int r0, int n_rows, uint16_t* dst,
                                          int wave, int lane) {
  using G = Geo<D>;
  const uint32_t skip = (uint32_t)min(r0, n_rows) * G::RB;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(g + (size_t)skip / 2, (uint32_t)n_rows * G::RB - skip);
  const int ld_row = lane / G::CPR, ld_chunk = lane % G::CPR;
  const int row = wave * G::RPL + ld_row;
  const uint32_t voff = (uint32_t)row * G::RB + 16u * (ld_chunk ^ G::swz(row));
#pragma unroll
  for (int i = 0; i < G::LPW; ++i)
    load_lds_16(rs, dst + (4 * i + wave) * 512, voff, (uint32_t)i * 4096);
}

// bf16 stores of one lane's C-layout accumulators (dims x rows, lane = row): 32 dims per tile
template <int D>
__device__ __forceinline__ void store_rowT(uint16_t* row_ptr, const f32x16 (&acc)[D / 32],
                                           float mul, int h) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const u32x2 w = {pack_bf16x2(acc[db][4 * g4 + 0] * mul, acc[db][4 * g4 + 1] * mul),
                       pack_bf16x2(acc[db][4 * g4 + 2] * mul, acc[db][4 * g4 + 3] * mul)};
      *(u32x2*)(row_ptr + 32 * db + 8 * g4 + 4 * h) = w;
    }
}

// The per-lane P and dS of one C tile from its scores s and dP values (both in place: s -> P,
// dp -> dS), given the reference (LSE in log2 units) and D of each element.
__device__ __forceinline__ void p_and_ds(float& s, float& dp, float c, float lse2, float dd) {
  const float p = fast_exp2(fmaf(s, c, -lse2));
  s = p;
  dp = p * (dp - dd);
}

// ---------------------------------------------------------------------------------------------
// dQ: workgroup = 4 waves = 128 query rows; 64-key blocks of K and V through LDS.
template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ O, const float* __restrict__ LSE, float* __restrict__ Ln,
    float* __restrict__ Dn, uint16_t* __restrict__ dQ,
    const int* __restrict__ seqlens, const uint16_t* __restrict__ bias, int bias_b, int bias_h,
    int Hq, int Hkv, int Nq, int Nk_cap, int nqt, float scale, float scale_log2) {
  constexpr int TILE = Geo<D>::TILE, NCB = Geo<D>::NCB, NDB = Geo<D>::NDB;
  __shared__ __attribute__((aligned(1024))) uint16_t kl0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t kl1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vl0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vl1[TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int BH = gridDim.x / nqt;
  const int bh = blockIdx.x % BH, qt = nqt - 1 - blockIdx.x / BH;  // heaviest blocks first
  const int b = bh / Hq, hq = bh - b * Hq, hkv = hq / (Hq / Hkv);
  // keys of this batch element: all Nk_cap rows of K/V, or the first seqlens[b] (clamped)
  const int Nk = seqlens ? min(max(seqlens[b], 0), Nk_cap) : Nk_cap;
  const int off = Nk - Nq;
  const int qw0 = qt * 128 + wave * 32, my_q = qw0 + l32;
  const uint16_t* kg = K + (size_t)(b * Hkv + hkv) * Nk_cap * D;
  const uint16_t* vg = V + (size_t)(b * Hkv + hkv) * Nk_cap * D;

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(Nq - 1, qt * 128 + 127) + off + 1);
  const int n_blk = kv_end > 0 ? (kv_end + BT - 1) / BT : 0;

  // additive bias (bf16 [bias_b, bias_h, Nq, Nk_cap], batch / head dims broadcast when 1), taken
  // off the row's reference in log2 units (bias log2e), which adds bias / scale to the scores.  A resource covers this
  // wave's 32 rows (rows past Nq read zero); a lane loads its row's 4-key groups, 8 bytes each.
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(
      BIAS ? bias + (((size_t)(bias_b == 1 ? 0 : b) * bias_h + (bias_h == 1 ? 0 : hq)) * Nq +
                     (size_t)min(qw0, Nq)) * Nk_cap
           : nullptr,
      BIAS ? (uint32_t)max(0, min(32, Nq - qw0)) * Nk_cap * 2 : 0u);
  const uint32_t b_lane = (uint32_t)l32 * Nk_cap * 2 + 8u * h;

  // Q and dO of this lane's query as the B operand (dims 16c + 8h .. +7), and O's same dims for
  // D = sum_d dO O: the lane's 8-dim dot products summed as a tree, then the partner lane's half
  u32x4 qf[NCB], gf[NCB];
  float dd;
  {
    const bool ok = my_q < Nq;
    const size_t row = (size_t)bh * Nq + min(my_q, Nq - 1);
    float part[NCB];
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      qf[c] = ok ? *(const u32x4*)(Q + row * D + 16 * c + 8 * h) : u32x4{0u, 0u, 0u, 0u};
      gf[c] = ok ? *(const u32x4*)(dO + row * D + 16 * c + 8 * h) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 o = ok ? *(const u32x4*)(O + row * D + 16 * c + 8 * h) : u32x4{0u, 0u, 0u, 0u};
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a += __uint_as_float(o[i] << 16) * __uint_as_float(gf[c][i] << 16);
        a += __uint_as_float(o[i] & 0xffff0000u) * __uint_as_float(gf[c][i] & 0xffff0000u);
      }
      part[c] = a;
    }
#pragma unroll
    for (int w = 1; w < NCB; w *= 2)
#pragma unroll
      for (int c = 0; c + w < NCB; c += 2 * w) part[c] += part[c + w];
    dd = part[0] + __shfl_xor(part[0], 32);
  }
  // the row's reference in log2 units, LSE log2e (+inf: no visible key, so every P is 0); the
  // row terms -D and -LSE / scale (-inf for such a row) go to the workspace for the dK/dV kernel
  float lse2 = INFINITY;
  if (my_q < Nq) {
    const size_t row = (size_t)bh * Nq + my_q;
    const float l = LSE[row];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    if (h == 0) {
      Dn[row] = -dd;
      Ln[row] = l == -INFINITY ? -INFINITY : -l / scale;
    }
  }

  const TileLanes tl = tile_lanes<D>(lane);
  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};

  if (n_blk > 0) {
    copy_tile<D>(kg, 0, Nk, kl0, wave, lane);
    copy_tile<D>(vg, 0, Nk, vl0, wave, lane);
  }
  // step t reads buffer BUF = t % 2 and copies block t + 1 into the other one; the buffers are
  // named at compile time so that the compiler sees that the copies and the reads touch
  // different arrays (otherwise it waits for the copies before the transposing reads)
  auto step = [&](auto buf_tag, int t) {
    constexpr int BUF = decltype(buf_tag)::value;
    const uint16_t* const kc = BUF ? kl1 : kl0;
    const uint16_t* const vc = BUF ? vl1 : vl0;
    wait_vmem();
    __syncthreads();  // block t is in LDS; the other buffers are free
    if (t + 1 < n_blk) {
      copy_tile<D>(kg, (t + 1) * BT, Nk, BUF ? kl0 : kl1, wave, lane);
      copy_tile<D>(vg, (t + 1) * BT, Nk, BUF ? vl0 : vl1, wave, lane);
    }
    if (qw0 >= Nq || (CAUSAL && t * BT > qw0 + 31 + off)) return;
    // S^T = K Q^T and dP^T = V dO^T, 32 keys at a time (keys 32 kb + 8 (r >> 2) + 4 h + (r & 3)
    // of this query), each half turned into its dS^T operands before the next is computed
    const int k0 = t * BT;
    const bool need = (k0 + BT > Nk) || (CAUSAL && (k0 + BT - 1 > qw0 + off));
    const int lim = CAUSAL ? min(Nk - 1, my_q + off) : Nk - 1;
    u32x4 pb[4];
    u32x2 bw[8];  // bias of keys k0 + 32 (i >> 2) + 8 (i & 3) + 4 h .. +3, this lane's row
    if constexpr (BIAS) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        bw[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                    brs, (int)(b_lane + (uint32_t)(32 * (i >> 2) + 8 * (i & 3)) * 2), k0 * 2, 0));
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      // the operands of slice c are read PF slices ahead of their products into a ring, and the
      // scheduling fences keep that distance: left to itself the compiler reads each operand
      // right before its product and waits for it there
      constexpr int PF = 3, NR = PF + 1;
      u32x4 ak[NR], av[NR];
#pragma unroll
      for (int c = 0; c < PF; ++c) {
        ak[c] = read_row<D>(kc, tl.row_base, kb, c);
        av[c] = read_row<D>(vc, tl.row_base, kb, c);
      }
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        if (c + PF < NCB) {
          ak[(c + PF) % NR] = read_row<D>(kc, tl.row_base, kb, c + PF);
          av[(c + PF) % NR] = read_row<D>(vc, tl.row_base, kb, c + PF);
        }
        s = mfma32x32x16(ak[c % NR], qf[c], s);
        dp = mfma32x32x16(av[c % NR], gf[c], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float s0 = s[r], s1 = s[r + 1], d0 = dp[r], d1 = dp[r + 1];
        float l0 = lse2, l1 = lse2;
        if constexpr (BIAS) {  // bias · log2e taken off the reference (bias / scale in scores)
          const uint32_t w = bw[4 * kb + (r >> 2)][(r >> 1) & 1];
          l0 = fmaf(__uint_as_float(w << 16), -kLog2e, lse2);
          l1 = fmaf(__uint_as_float(w & 0xffff0000u), -kLog2e, lse2);
        }
        p_and_ds(s0, d0, scale_log2, l0, dd);
        p_and_ds(s1, d1, scale_log2, l1, dd);
        const int j = 16 * kb + r;
        pb[j >> 3][(j >> 1) & 3] = pack_bf16x2(d0, d1);
      }
      if (need) {  // clear the bf16 halves of dS entries past the last visible key
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3), j = 16 * kb + r;
          pb[j >> 3][(j >> 1) & 3] &= (key <= lim ? 0x0000ffffu : 0u) | (key + 1 <= lim ? 0xffff0000u : 0u);
        }
      }
    }
    // dQ^T += K^T dS^T, 16 keys at a time
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = mfma32x32x16(read_tr<D>(kc, tl.tr_base, 16 * g, db), pb[g], acc[db]);
  };
  for (int t = 0; t < n_blk; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < n_blk) step(std::integral_constant<int, 1>{}, t + 1);
  }
  if (my_q < Nq) store_rowT<D>(dQ + ((size_t)bh * Nq + my_q) * D, acc, scale, h);
}

// ---------------------------------------------------------------------------------------------
// dK and dV: workgroup = 8 waves for 128 keys; 64-row blocks of Q, dO and their row terms go
// through LDS once for all of them, for every query head of the K/V head's group.  Waves w and
// w + 4 share 32 keys: wave w computes S = Q K^T, turns it into P and accumulates dV^T += dO^T P;
// wave w + 4 computes dP = dO V^T, takes P from wave w through LDS and accumulates
// dK^T += Q^T dS.  So every wave runs two of the four products per block and holds one operand
// set and one accumulator set, and the two waves of a SIMD carry equal loads.  The dK waves work
// one block behind the dV waves (the P of block t is read in step t + 1), so one barrier per step
// orders everything: Q / dO / reference blocks are triple-buffered, P double-buffered.
template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ Ln, const float* __restrict__ Dn, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, const int* __restrict__ seqlens, const uint16_t* __restrict__ bias,
    int bias_b, int bias_h, int Hq, int Hkv, int Nq, int Nk_cap, int nkt, float scale,
    float scale_log2) {
  constexpr int TILE = Geo<D>::TILE, NCB = Geo<D>::NCB, NDB = Geo<D>::NDB;
  __shared__ __attribute__((aligned(1024))) uint16_t qls[3][TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t gls[3][TILE];
  __shared__ __attribute__((aligned(16))) float sls[3][2 * BT];  // -LSE / scale, then -D
  // P of each wave pair as packed bf16 operands: [buffer][pair][operand i][lane], 16 bytes each,
  // so that a wave's 16-byte stores and loads of one operand cover 1 KB contiguously
  __shared__ __attribute__((aligned(1024))) u32x4 pls[2][4 * 4 * 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const bool do_k = wave >= 4;
  const int pair = wave & 3;
  const int BHk = gridDim.x / nkt;
  const int bhk = blockIdx.x % BHk, kt = blockIdx.x / BHk;
  const int b = bhk / Hkv, hkv = bhk - b * Hkv, G = Hq / Hkv;
  // keys of this batch element (as in the dQ kernel); keys past them keep zero gradients
  const int Nk = seqlens ? min(max(seqlens[b], 0), Nk_cap) : Nk_cap;
  const int off = Nk - Nq;
  const int kw0 = kt * 128 + pair * 32, my_k = kw0 + l32;

  // this lane's key row as the B operand of the wave's first product: K (for S) or V (for dP)
  u32x4 bf[NCB];
  {
    const bool ok = my_k < Nk;
    const uint16_t* row =
        (do_k ? V : K) + ((size_t)bhk * Nk_cap + min(my_k, max(Nk - 1, 0))) * D;
#pragma unroll
    for (int c = 0; c < NCB; ++c)
      bf[c] = ok ? *(const u32x4*)(row + 16 * c + 8 * h) : u32x4{0u, 0u, 0u, 0u};
  }

  // query blocks that see any key of this workgroup: rows q with q + off >= kt * 128
  const int q_first = CAUSAL ? max(0, kt * 128 - off) : 0;
  const int qb0 = q_first / BT, nqb = (Nq + BT - 1) / BT;
  const int per_head = max(0, nqb - qb0);
  const int n_steps = kt * 128 < Nk ? G * per_head : 0;  // no key of this tile exists: zeros

  auto stage = [&](int step, int buf) {
    const int g = step / per_head, qb = qb0 + step - g * per_head;
    const size_t bh = (size_t)b * Hq + hkv * G + g;
    if (wave < 4)  // waves 0-3 copy the Q block, waves 4-7 the dO block
      copy_tile<D>(Q + bh * Nq * D, qb * BT, Nq, qls[buf], wave, lane);
    else
      copy_tile<D>(dO + bh * Nq * D, qb * BT, Nq, gls[buf], wave - 4, lane);
    if (wave == 0) {  // 64 -LSE / scale then 64 -D, four bytes per lane; rows past Nq read zero
      const int q = qb * BT;
      const uint32_t n = (uint32_t)max(0, Nq - q) * 4;
      load_lds_4(make_rsrc(Ln + bh * Nq + min(q, Nq), n), sls[buf], (uint32_t)lane * 4);
      load_lds_4(make_rsrc(Dn + bh * Nq + min(q, Nq), n), sls[buf] + BT, (uint32_t)lane * 4);
    }
  };

  const TileLanes tl = tile_lanes<D>(lane);
  f32x16 acc[NDB];  // dK^T or dV^T of this wave's keys
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};

  if (n_steps > 0) stage(0, 0);
  // step t: the dV waves take block t (buffer t % 3), the dK waves block t - 1
  for (int t = 0, bc = 0; t <= n_steps; ++t, bc = bc == 2 ? 0 : bc + 1) {
    wait_vmem();
    __syncthreads();  // block t is in LDS, so is the P of block t - 1; buffer (t + 1) % 3 is free
    if (t + 1 < n_steps) stage(t + 1, bc == 2 ? 0 : bc + 1);
    const int blk = do_k ? t - 1 : t;
    if (blk < 0 || blk >= n_steps) continue;
    const int bb = do_k ? (bc == 0 ? 2 : bc - 1) : bc;
    const uint16_t* qc = qls[bb];
    const uint16_t* gc = gls[bb];
    const float* sc = sls[bb];
    u32x4* const pw = pls[blk & 1] + pair * 4 * 64 + lane;  // this lane's operand slots (stride 64)
    const int q0 = (qb0 + blk % per_head) * BT;
    if (kw0 >= Nk || (CAUSAL && q0 + BT - 1 + off < kw0)) continue;  // nothing visible
    // additive bias of this lane's key for the block's 64 query rows (dV waves only: the dK
    // waves take P from them), entry 16 half + 4 g4 + e for row 32 half + 8 g4 + 4 h + e; a
    // resource over the block's rows (rows past Nq read zero), requested before the first product
    uint32_t bq[32];
    if constexpr (BIAS) {
      if (!do_k) {
        const int g = blk / per_head;
        const size_t row0 =
            (((size_t)(bias_b == 1 ? 0 : b) * bias_h + (bias_h == 1 ? 0 : hkv * G + g)) * Nq +
             (size_t)q0) * Nk_cap;
        const __amdgpu_buffer_rsrc_t brs =
            make_rsrc(bias + row0, (uint32_t)max(0, min(BT, Nq - q0)) * Nk_cap * 2);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const uint32_t qrel = 32 * (i >> 4) + 8 * ((i >> 2) & 3) + 4 * h + (i & 3);
          bq[i] = __builtin_amdgcn_raw_buffer_load_b16(brs, (int)((qrel * Nk_cap + my_k) * 2), 0, 0);
        }
      }
    }
    // first product for both 32-row halves, interleaved: S = Q K^T or dP = dO V^T; half j holds
    // queries q0 + 32 j + 8 (r >> 2) + 4 h + (r & 3) of this key.  The accumulators start at the
    // rows' negated terms, so they end as S - LSE / scale (dV waves) or dP - D (dK waves).
    f32x16 r2[2];
    {
      const float* rb = sc + (do_k ? BT : 0);
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 v4 = *(const f32x4*)(rb + 32 * half + 8 * g4 + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) r2[half][4 * g4 + e] = v4[e];
        }
    }
    u32x4 pw4[4];  // the dK waves' P of this block, from the pair's dV wave
    if (do_k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pw4[i] = pw[64 * i];
    }
    {
      // operands read PF slices ahead into a ring, as in the dQ kernel
      const uint16_t* xa = do_k ? gc : qc;
      constexpr int PF = 2, NR = PF + 1;
      u32x4 ar[NR][2];
#pragma unroll
      for (int c = 0; c < PF; ++c)
#pragma unroll
        for (int half = 0; half < 2; ++half) ar[c][half] = read_row<D>(xa, tl.row_base, half, c);
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        if (c + PF < NCB) {
#pragma unroll
          for (int half = 0; half < 2; ++half)
            ar[(c + PF) % NR][half] = read_row<D>(xa, tl.row_base, half, c + PF);
        }
#pragma unroll
        for (int half = 0; half < 2; ++half)
          r2[half] = mfma32x32x16(ar[c % NR][half], bf[c], r2[half]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    u32x4 pb[4];  // P (dV) or dS (dK) as the B operand of the second product, 16 queries each
    if (!do_k) {
      // P = 2^((S - LSE / scale) scale log2e), zero outside the causal / valid range, published
      // for the pair's dK wave (rows past Nq read a term of 0 and are masked)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qh0 = q0 + 32 * half;
        const bool need = (qh0 + 32 > Nq) || (kw0 + 32 > Nk) || (CAUSAL && kw0 + 31 > qh0 + off);
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float p[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float x = r2[half][r + e] * scale_log2;
            if constexpr (BIAS)  // bias · log2e added to the exponent (bias / scale in scores)
              x = fmaf(__uint_as_float(bq[16 * half + r + e] << 16), kLog2e, x);
            p[e] = fast_exp2(x);
          }
          const int j = 16 * half + r;
          pb[j >> 3][(j >> 1) & 3] = pack_bf16x2(p[0], p[1]);
        }
        if (need) {  // clear the bf16 halves of masked entries
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const int q = qh0 + 8 * (r >> 2) + 4 * h + (r & 3), j = 16 * half + r;
            const bool ok0 = q < Nq && my_k < Nk && (!CAUSAL || my_k <= q + off);
            const bool ok1 = q + 1 < Nq && my_k < Nk && (!CAUSAL || my_k <= q + 1 + off);
            pb[j >> 3][(j >> 1) & 3] &= (ok0 ? 0x0000ffffu : 0u) | (ok1 ? 0xffff0000u : 0u);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[64 * i] = pb[i];
    } else {
      // dS = P (dP - D) from the pair's P of this block (zero wherever the pair is masked)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int j = 16 * half + r;
          const uint32_t w = pw4[j >> 3][(j >> 1) & 3];
          pb[j >> 3][(j >> 1) & 3] = pack_bf16x2(__uint_as_float(w << 16) * r2[half][r],
                                                 __uint_as_float(w & 0xffff0000u) * r2[half][r + 1]);
        }
    }
    // dK^T += Q^T dS or dV^T += dO^T P, 16 queries at a time, at raised priority so that the
    // SIMD's other wave fills the gaps between these products with its vector work
    const uint16_t* at = do_k ? qc : gc;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = mfma32x32x16(read_tr<D>(at, tl.tr_base, 16 * g, db), pb[g], acc[db]);
    __builtin_amdgcn_s_setprio(0);
  }
  if (my_k < Nk_cap)
    store_rowT<D>((do_k ? dK : dV) + ((size_t)bhk * Nk_cap + my_k) * D, acc, do_k ? scale : 1.f,
                  h);
}

template <int D, bool CAUSAL, bool BIAS>
hipError_t launch(const void* q, const void* k, const void* v, const void* out, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, float* ws_d, const int* seqlens,
                  const void* bias, int bias_b, int bias_h, const AttnShape& s, float scale,
                  hipStream_t stream) {
  const long long rows = (long long)s.B * s.Hq * s.Nq;
  float* const ws_l2 = ws_d + rows;  // the workspace holds -D, then -LSE / scale
  const int nqt = (s.Nq + 127) / 128, nkt = (s.Nk + 127) / 128;
  const long long g_dq = (long long)s.B * s.Hq * nqt, g_kv = (long long)s.B * s.Hkv * nkt;
  if (g_dq > 0x7fffffffLL || g_kv > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipError_t e = hipSuccess;
  // the dQ kernel first: it also writes the row terms the dK/dV kernel reads
  if (g_dq > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, BIAS>), dim3((unsigned)g_dq), dim3(256), 0,
                       stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)dout, (const uint16_t*)out, lse, ws_l2, ws_d,
                       (uint16_t*)dq, seqlens, (const uint16_t*)bias, bias_b, bias_h, s.Hq, s.Hkv,
                       s.Nq, s.Nk, nqt, scale, scale * kLog2e);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (g_kv > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, BIAS>), dim3((unsigned)g_kv), dim3(512), 0,
                       stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)dout, (const float*)ws_l2, (const float*)ws_d, (uint16_t*)dk,
                       (uint16_t*)dv, seqlens, (const uint16_t*)bias, bias_b, bias_h, s.Hq, s.Hkv,
                       s.Nq, s.Nk, nkt, scale, scale * kLog2e);
    e = hipGetLastError();
  }
  return e;
}

template <int D, bool CAUSAL>
hipError_t launch_b(const void* q, const void* k, const void* v, const void* out, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, float* ws_d,
                    const int* seqlens, const void* bias, int bias_b, int bias_h,
                    const AttnShape& s, float scale, hipStream_t stream) {
  return bias ? launch<D, CAUSAL, true>(q, k, v, out, lse, dout, dq, dk, dv, ws_d, seqlens, bias,
                                        bias_b, bias_h, s, scale, stream)
              : launch<D, CAUSAL, false>(q, k, v, out, lse, dout, dq, dk, dv, ws_d, seqlens,
                                         nullptr, 1, 1, s, scale, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* ws_d, const int* seqlens, const void* bias, int bias_b,
                           int bias_h, const AttnShape& s, float scale, bool causal,
                           hipStream_t stream) {
  if (s.d == 128)
    return causal ? launch_b<128, true>(q, k, v, out, lse, dout, dq, dk, dv, ws_d, seqlens, bias,
                                        bias_b, bias_h, s, scale, stream)
                  : launch_b<128, false>(q, k, v, out, lse, dout, dq, dk, dv, ws_d, seqlens, bias,
                                         bias_b, bias_h, s, scale, stream);
  return causal ? launch_b<64, true>(q, k, v, out, lse, dout, dq, dk, dv, ws_d, seqlens, bias,
                                     bias_b, bias_h, s, scale, stream)
                : launch_b<64, false>(q, k, v, out, lse, dout, dq, dk, dv, ws_d, seqlens, bias,
                                      bias_b, bias_h, s, scale, stream);
}

}  // namespace fa
