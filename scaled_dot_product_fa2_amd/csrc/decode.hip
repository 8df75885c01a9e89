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
//   * split kernel: one workgroup per (batch, KV head, row group of 16, split).  The 16 "query"
//     columns of the MFMA are the Hq/Hkv query heads x Nq rows that share the KV head, so every
//     K/V byte of the split is read from HBM exactly once.  A grid with at least one workgroup
//     per SIMD and row groups at least half full uses one-wave workgroups (all resident at once,
//     one wave per SIMD); other grids use four waves per workgroup.  Each wave streams its own
//     32-key blocks (block w, w+NW, ...) with non-temporal 16-byte buffer loads whose range ends
//     at the split (later keys read as zero), keeps the next block (four waves) or two (a lone
//     wave) in flight in registers, stages the current one in a wave-private LDS slice, and keeps
//     its own running (m, l, Oᵀ); four waves are merged through LDS at the end into one locally
//     normalised partial, a lone wave stores its own.
//   * Products on v_mfma_f32_16x16x32_bf16: Sᵀ = K·Qᵀ, then Oᵀ += Vᵀ·Pᵀ with Pᵀ taken straight
//     from the score registers and Vᵀ from the transposing LDS read.
//   * combine kernel: one wave per (batch, query head, row); the split metadata is read by all
//     lanes at once and the partial rows are accumulated in a fixed split order, so the result
//     is deterministic.
//   * When the (batch, KV head) pairs are a multiple of 8 (the XCD count), every workgroup of
//     one pair, in both kernels, runs on the same XCD, so the combine reads the partials that
//     the split wrote from that XCD's L2 instead of from memory.
#include "fa_device.h"
#include "fa_kernels.h"

#include <math.h>

#include <atomic>

namespace fa {

// Workspace of attn_decode_splitkv_noalloc, for callers that cannot allocate: a fixed array in
// the code object, one copy per device (each GPU the library runs on holds it until the process
// ends).  Host code never uses its name as an address (in host code the name is a host-side
// stand-in); the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {

constexpr long long kSimdCount = 1024;  // MI355X: 256 CUs x 4 SIMDs

template <int D, int NW_>
struct DecCfg {
  static constexpr int KB = 32;               // keys per wave block
  static constexpr int QC = 16;               // query columns per workgroup (MFMA N)
  static constexpr int NW = NW_;              // waves per workgroup (1 or 4)
  static constexpr int NT = 64 * NW;
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int NCH = KB * CPR / 64;   // chunks per lane per tensor per block
  static constexpr int WTILE = 2 * KB * D;    // one wave's K block + V block (bf16)
  static constexpr int OROW = D + 4;          // fp32 pitch of the cross-wave merge buffer
  static constexpr int STAGE_BYTES = NW * WTILE * 2;
  static constexpr int MERGE_BYTES = NW * QC * OROW * 4 + NW * QC * 3 * 4;
  static constexpr int SMEM = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
};

// LDS placement of a wave's staged block: rows unpadded, 16-byte chunks XOR-swizzled so that
// both read patterns are conflict-free on the 64 banks.  K operand reads take 16 consecutive
// rows at one chunk per cycle; the transposing V reads take 8 consecutive rows x 2 adjacent
// chunks per cycle.
template <int D>
__device__ __forceinline__ int dk_chunk(int row, int c) {
  return D == 128 ? (c ^ (row & 15)) : (c ^ ((row >> 1) & 7));
}
template <int D>
__device__ __forceinline__ int dv_chunk(int row, int c) {
  return D == 128 ? (c ^ ((row & 7) << 1)) : (c ^ (((row >> 1) & 3) << 1));
}

// Orders this wave's LDS writes before its later LDS reads of other lanes' data.  A wave's LDS
// operations complete in issue order, so only compiler reordering has to be prevented.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// max / sum over the four lanes {q, q+16, q+32, q+48} (every one of them gets the result)
__device__ __forceinline__ float quad_max(float x) {
  x = pair32_max(x);
  return fmaxf(x, __shfl_xor(x, 16));
}
__device__ __forceinline__ float quad_sum(float x) {
  x = pair32_sum(x);
  return x + __shfl_xor(x, 16);
}

template <int D, bool CAUSAL, bool BIAS, int NW>
__global__ __launch_bounds__(64 * NW, NW == 1 ? 1 : 2) void decode_split_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ wsO, float* __restrict__ wsML,
    const int* __restrict__ seqlens, const uint16_t* __restrict__ bias, int bias_b, int bias_h,
    int Hq, int Hkv, int Nq, int Nk_cap, int S, int L, int nrg, float scale, float scale_log2,
    int xcd_pairs) {
  using C = DecCfg<D, NW>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, l16 = lane & 15;  // 16-lane group, query column
  // workgroup -> (batch, KV head, row group, split).  Workgroup n runs on XCD n mod 8; when the
  // (batch, KV head) pairs are a multiple of 8, all workgroups of one pair go to one XCD (pair p
  // to XCD p mod 8), so the combine kernel, which maps its rows the same way, reads the partials
  // from that XCD's L2.  Otherwise the split index runs fastest.
  int s, rg, hkv, b;
  if (xcd_pairs) {
    const int per = nrg * S, j = blockIdx.x >> 3;
    const int pair = (j / per) * 8 + (blockIdx.x & 7), w = j % per;
    rg = w / S;
    s = w % S;
    hkv = pair % Hkv;
    b = pair / Hkv;
  } else {
    int n = blockIdx.x;
    s = n % S;
    n /= S;
    rg = n % nrg;
    n /= nrg;
    hkv = n % Hkv;
    b = n / Hkv;
  }
  const int G = Hq / Hkv, R = G * Nq;
  // keys of this batch element: all Nk_cap rows of K/V, or the first seqlens[b] (clamped); the
  // split chunks are those of the capacity, clipped to it
  const int Nk = seqlens ? min(max(seqlens[b], 0), Nk_cap) : Nk_cap;
  const int off = Nk - Nq;

  // this lane's query column: row r of the KV head's group = (query head offset g, position qi)
  const int r = rg * C::QC + l16;
  const bool row_ok = r < R;
  const int g = row_ok ? r / Nq : 0;
  const int qi = row_ok ? r - g * Nq : 0;
  const int hq = hkv * G + g;

  const int ks0 = min(s * L, Nk), ks1 = min(ks0 + L, Nk);
  const int nkb = (ks1 - ks0 + C::KB - 1) / C::KB;
  const int lim = CAUSAL ? min(ks1 - 1, qi + off) : ks1 - 1;  // last visible key of this row

  // buffer resources covering exactly this split's keys: rows past the split read as zero
  const size_t split_off = (((size_t)b * Hkv + hkv) * Nk_cap + ks0) * D;
  const uint32_t split_bytes = (uint32_t)(ks1 - ks0) * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + split_off, split_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + split_off, split_bytes);
  // additive bias (bf16 [bias_b, bias_h, Nq, Nk_cap], broadcast over batch / heads when 1): a
  // lane needs keys key .. key+3 of its own row, key = ks0 + 32kb + 16hh + 4grp, for each of two
  // groups per block, loaded with the block's K/V.  Every load is an aligned 8-byte unit of four
  // keys [4u, 4u + 4): rows start 8-byte aligned (16-byte aligned base, Nk_cap % 4 == 0), so such
  // a unit never crosses the end of the row.  key is congruent to the split start mod 4, so the
  // misalignment a = ks0 mod 4 is the same for the whole workgroup: for a == 0 the group is one
  // unit; otherwise it spans two units, the second loaded only when a key it supplies is inside
  // the split, and the four keys are shifted out of the pair.  Keys at or past the split end
  // are masked, so whatever a unit holds there is never used.
  const uint16_t* brow =
      BIAS ? bias + (((size_t)(bias_b == 1 ? 0 : b) * bias_h + (bias_h == 1 ? 0 : hq)) * Nq + qi) *
                        Nk_cap
           : nullptr;
  const int bias_mis = ks0 & 3;  // misalignment of every group of this workgroup, in keys
  const float inv_scale = 1.f / scale;
  uint16_t* kls = (uint16_t*)smem + wave * C::WTILE;
  uint16_t* vls = kls + C::KB * D;

  // K/V blocks travel HBM -> registers (16-byte coalesced loads, two blocks in flight per wave)
  // -> this wave's LDS slice -> MFMA operands.  Chunk i of a lane is byte
  // (32 kb + lane / CPR + i * 64 / CPR) * 2D + (lane % CPR) * 16 of the split.
  const uint32_t lane_off = (uint32_t)(lane / C::CPR) * (D * 2) + (uint32_t)(lane % C::CPR) * 16;
  auto gload = [&](u32x4 (&kst)[C::NCH], u32x4 (&vst)[C::NCH], u32x2 (&bst)[2], int kb) {
    const uint32_t voff = lane_off + (uint32_t)(C::KB * kb) * (D * 2);
#pragma unroll
    for (int i = 0; i < C::NCH; ++i) {
      kst[i] = load_16_stream(krs, voff, i * 1024u);
      vst[i] = load_16_stream(vrs, voff, i * 1024u);
    }
    if constexpr (BIAS) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int unit = ks0 + C::KB * kb + 16 * hh + 4 * grp - bias_mis;  // a multiple of 4
        uint64_t lo = 0, hi = 0;
        if (row_ok && unit + bias_mis < ks1) lo = *(const uint64_t*)(brow + unit);
        if (row_ok && bias_mis != 0 && unit + 4 < ks1) hi = *(const uint64_t*)(brow + unit + 4);
        const uint64_t w = bias_mis == 0 ? lo : (lo >> (16 * bias_mis)) | (hi << (64 - 16 * bias_mis));
        bst[hh] = __builtin_bit_cast(u32x2, w);
      }
    }
  };
  auto swrite = [&](const u32x4 (&kst)[C::NCH], const u32x4 (&vst)[C::NCH]) {
#pragma unroll
    for (int i = 0; i < C::NCH; ++i) {
      const int ci = lane + 64 * i;
      const int row = ci / C::CPR, c = ci % C::CPR;
      *(u32x4*)(kls + row * D + 8 * dk_chunk<D>(row, c)) = kst[i];
      *(u32x4*)(vls + row * D + 8 * dv_chunk<D>(row, c)) = vst[i];
    }
  };

  // blocks in flight per wave: two for a lone wave, one for each of four (a second or third one
  // there measured 1-9% slower, as more concurrent streams compete for the DRAM pages)
  constexpr int NB = C::NW == 1 ? 2 : 1;
  u32x4 kst[NB][C::NCH], vst[NB][C::NCH];
  u32x2 bst[NB][2];
  const int kb0 = wave;
  // The split's blocks are taken in a rotated order, block (j + rot) mod nkb at step j, with the
  // rotation varying over splits and (batch, KV head) pairs.  Every split starts at a multiple
  // of its length from the tensor's base, so without it all workgroups request the same offset
  // within their splits at the same time, which lands on fewer memory channels; how much that
  // costs depends on where the K/V allocations fall (GQA decode at Nq = 4: 47.8 -> 46.9 us,
  // and 51.7 -> 48.8 us with other allocations made first).  The order changes only the
  // summation order of the split's partial.
  const int rot =
      nkb > 0 ? (int)((7u * (unsigned)s + 5u * (unsigned)(b * Hkv + hkv)) % (unsigned)nkb) : 0;
  auto phys = [&](int j) { const int k = j + rot; return k >= nkb ? k - nkb : k; };
#pragma unroll
  for (int u = 0; u < NB; ++u)
    if (kb0 + u * C::NW < nkb) gload(kst[u], vst[u], bst[u], phys(kb0 + u * C::NW));

  // Qᵀ as the B operand of Sᵀ = K·Qᵀ (16x16x32): lane holds query column l16, head-dim slots
  // 32c + 8grp .. +7.
  u32x4 qf[D / 32];
  {
    const uint16_t* qrow = Q + (((size_t)b * Hq + hq) * Nq + qi) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      qf[c] = row_ok ? *(const u32x4*)(qrow + 32 * c + 8 * grp) : u32x4{0u, 0u, 0u, 0u};
  }

  f32x4 oacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{};
  // m_run: the lazily moved reference the exponents use; m_true: the exact running max, which
  // the stored metadata reports
  float m_run = -INFINITY, m_true = -INFINITY, l_run = 0.f;
  const int tr_j = l16 >> 2, tr_t = l16 & 3;

  // one staged block: scores, masked online softmax, Oᵀ += Vᵀ·Pᵀ
  auto compute = [&](int kb, const u32x2 (&bst)[2]) {
    const int k0 = ks0 + C::KB * kb;
    // Sᵀ (32 keys x 16 queries) in two 16-key halves: sc[h][i] is key k0 + 16h + 4grp + i
    f32x4 sc[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 16 * hh + l16;
      sc[hh] = f32x4{};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const u32x4 a = *(const u32x4*)(kls + row * D + 8 * dk_chunk<D>(row, 4 * c + grp));
        sc[hh] = mfma16x16x32(a, qf[c], sc[hh]);
      }
    }
    if constexpr (BIAS) {  // in score units, before the mask
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = bst[hh][i >> 1];
          sc[hh][i] += __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16)) * inv_scale;
        }
    }
    if (k0 + C::KB - 1 > lim) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k0 + 16 * hh + 4 * grp + i > lim) sc[hh][i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = quad_max(mx);
    m_true = fmaxf(m_true, mx);
    const bool grow = (mx - m_run) * scale_log2 > kLazyLog2;  // lazy reference max, as in prefill
    const float m_next = grow ? mx : m_run;
    const float alpha = grow ? fast_exp2((m_run - m_next) * scale_log2) : 1.f;
    if (wave_any(grow && m_run != -INFINITY)) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
    }
    m_run = m_next;
    const float mb = (m_run == -INFINITY ? 0.f : m_run) * scale_log2;
    float rs = 0.f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(fmaf(sc[hh][i], scale_log2, -mb));
        sc[hh][i] = p;
        rs += p;
      }
    l_run = l_run * alpha + rs;  // this lane group's keys; the four groups are summed at the end
    // Pᵀ (32 keys x 16 queries) as the B operand: slot 8grp + t is key 4grp + t (t < 4) or
    // 16 + 4grp + t - 4, matching the two transposing reads below.
    const u32x4 pb = {pack_bf16x2(sc[0][0], sc[0][1]), pack_bf16x2(sc[0][2], sc[0][3]),
                      pack_bf16x2(sc[1][0], sc[1][1]), pack_bf16x2(sc[1][2], sc[1][3])};
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int c = 2 * db + (tr_t >> 1), within = 4 * (tr_t & 1);
      const int r0 = 4 * grp + tr_j, r1 = r0 + 16;
      const bf16x8 a = lds_read_tr16_pair(vls + r0 * D + 8 * dv_chunk<D>(r0, c) + within,
                                          vls + r1 * D + 8 * dv_chunk<D>(r1, c) + within);
      oacc[db] = mfma16x16x32(a, pb, oacc[db]);
    }
  };

  // a block's registers are refilled with the block NB further on as soon as it is in LDS, so
  // the loads land while this block and the next NB - 1 are computed
  for (int kb = kb0; kb < nkb; kb += NB * C::NW) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int kbu = kb + u * C::NW;
      if (kbu < nkb) {
        swrite(kst[u], vst[u]);
        wave_lds_sync();
        const u32x2 bc[2] = {bst[u][0], bst[u][1]};
        if (kbu + NB * C::NW < nkb) gload(kst[u], vst[u], bst[u], phys(kbu + NB * C::NW));
        compute(phys(kbu), bc);
        wave_lds_sync();  // this block's LDS reads precede the next block's writes
      }
    }
  }

  const float l_tot = quad_sum(l_run);
  if constexpr (C::NW == 1) {
    // the wave is the whole split: the exact max M of its keys and the sum against M give the
    // metadata, and Oᵀ / l (both against the reference max) is the locally normalised partial,
    // stored straight from the accumulator layout (lane (l16, grp), register i of tile db holds
    // head-dim slot 16 db + 4 grp + i of query column l16)
    if (row_ok) {
      const float M = l_tot > 0.f ? m_true : -INFINITY;
      const float ew = l_tot > 0.f ? fast_exp2((m_run - M) * scale_log2) : 0.f;
      const float Lsum = ew * l_tot;
      const float f = Lsum > 0.f ? ew * (1.f / Lsum) : 0.f;
      const size_t slot = (((size_t)b * Hq + hq) * Nq + qi) * S + s;
      float* dst = wsO + slot * D + 4 * grp;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) *(f32x4*)(dst + 16 * db) = oacc[db] * f;
      if (grp == 0) {
        wsML[slot * 2 + 0] = Lsum > 0.f ? M * scale : -INFINITY;
        wsML[slot * 2 + 1] = Lsum;
      }
    }
    return;
  }

  // merge the waves' (m, l, Oᵀ) into one locally normalised partial for the split
  __syncthreads();
  float* ocb = (float*)smem;                 // [NW][QC][OROW] unnormalised Oᵀ rows
  float* mlb = ocb + C::NW * C::QC * C::OROW;  // [NW][QC][3]: exact max, reference max, sum
                                             // (score units; the sum is against the reference)
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    *(f32x4*)(ocb + (wave * C::QC + l16) * C::OROW + 16 * db + 4 * grp) = oacc[db];
  if (grp == 0) {
    mlb[(wave * C::QC + l16) * 3 + 0] = m_true;
    mlb[(wave * C::QC + l16) * 3 + 1] = m_run;
    mlb[(wave * C::QC + l16) * 3 + 2] = l_tot;
  }
  __syncthreads();

  constexpr int TPQ = C::NT / C::QC;  // threads per query column in the merge
  constexpr int DE = D / TPQ;         // head-dim elements per merging thread
  const int qr = tid / TPQ, ch = tid % TPQ;
  const int rr = rg * C::QC + qr;
  if (rr < R) {
    const int g2 = rr / Nq, qi2 = rr - g2 * Nq;
    const int hq2 = hkv * G + g2;
    // M = exact max of the split; each wave's sum and accumulator are re-expressed against it
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < C::NW; ++w)
      if (mlb[(w * C::QC + qr) * 3 + 2] > 0.f) M = fmaxf(M, mlb[(w * C::QC + qr) * 3]);
    float ew[C::NW];
    float Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) {
      const float lw = mlb[(w * C::QC + qr) * 3 + 2];
      ew[w] = lw > 0.f ? fast_exp2((mlb[(w * C::QC + qr) * 3 + 1] - M) * scale_log2) : 0.f;
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
        o += ew[w] * *(const f32x4*)(ocb + (w * C::QC + qr) * C::OROW + ch * DE + e);
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

// One wave per output row (batch, query head, position).  The first 16 partial rows are
// requested before anything else, so their latency overlaps the metadata pass; lane s reads the
// (m, l) of split s (64 splits per pass), the weights w_s = l_s exp(m_s - M) are then broadcast
// lane by lane, and the rows are accumulated in split order (deterministic).
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ wsO,
                                                           const float* __restrict__ wsML,
                                                           uint16_t* __restrict__ O,
                                                           float* __restrict__ LSE, int rows,
                                                           int S, int xcd_pairs, int R) {
  constexpr int E = D / 64;  // head-dim elements per lane
  constexpr int CH = 16;     // partial rows in flight per lane
  typedef float vecE __attribute__((ext_vector_type(E)));
  const int lane = threadIdx.x;
  // the R rows of a (batch, KV head) pair are consecutive; with the split kernel's XCD mapping,
  // pair p's rows run on XCD p mod 8 as well
  int row = blockIdx.x;
  if (xcd_pairs) {
    const int j = row >> 3;
    row = ((j / R) * 8 + (row & 7)) * R + j % R;
  }
  if (row >= rows) return;
  const f32x2* ml = (const f32x2*)(wsML + (size_t)row * S * 2);
  const float* src = wsO + (size_t)row * S * D + lane * E;

  vecE o[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) o[j] = (j < S) ? *(const vecE*)(src + (size_t)j * D) : vecE{};

  float M = -INFINITY;  // exact max over the splits that saw a key
  for (int s0 = 0; s0 < S; s0 += 64) {
    const f32x2 v = (s0 + lane < S) ? ml[s0 + lane] : f32x2{-INFINITY, 0.f};
    M = fmaxf(M, v[1] > 0.f ? v[0] : -INFINITY);
  }
  M = wave_max(M);

  vecE acc = vecE{};
  float W = 0.f;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int n = min(64, S - s0);
    const f32x2 v = (lane < n) ? ml[s0 + lane] : f32x2{-INFINITY, 0.f};
    const float w = v[1] > 0.f ? v[1] * fast_exp2((v[0] - M) * kLog2e) : 0.f;
    W += w;
    for (int c0 = 0; c0 < n; c0 += CH) {
      if (s0 + c0 > 0) {
#pragma unroll
        for (int j = 0; j < CH; ++j)
          o[j] = (c0 + j < n) ? *(const vecE*)(src + (size_t)(s0 + c0 + j) * D) : vecE{};
      }
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        if (c0 + j < n) {
          const float wj = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), c0 + j));
          acc += wj * o[j];
        }
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

template <int D, bool CAUSAL, bool BIAS>
hipError_t launch(const void* q, const void* k, const void* v, void* out, float* lse,
                  float* ws_o, float* ws_ml, const int* seqlens, const void* bias, int bias_b,
                  int bias_h, const AttnShape& sh, float scale, int S, hipStream_t stream) {
  constexpr int QC = DecCfg<D, 1>::QC;
  const int L = (sh.Nk + S - 1) / S;
  const int R = (sh.Hq / sh.Hkv) * sh.Nq;
  const int nrg = (R + QC - 1) / QC;
  const long long blocks = (long long)sh.B * sh.Hkv * nrg * S;
  const long long rows = (long long)sh.B * sh.Hq * sh.Nq;
  if (blocks > 0x7fffffffLL || rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int xcd_pairs = ((long long)sh.B * sh.Hkv) % 8 == 0 ? 1 : 0;
  // One wave per split when the grid has a workgroup for every SIMD (256 CUs x 4, all resident
  // at once) and at least half of a row group's 16 query columns are in use; otherwise four
  // waves per split, whose LDS merge is cheap with few columns and which fill the chip on small
  // grids.  Measured on the GQA decode workloads (1024 workgroups, four-wave vs one-wave):
  // Nq = 4 (16 columns) 49.4-50.0 vs 47.9-48.0 us, with a bias 53.0 vs 51.0; Nq = 1 (4 columns)
  // 45.4 vs 46.2, with a bias 47.9 vs 49.6.
  if (blocks >= kSimdCount && min(R, QC) >= QC / 2)
    hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL, BIAS, 1>), dim3((unsigned)blocks),
                       dim3(64), 0, stream, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, ws_o, ws_ml, seqlens, (const uint16_t*)bias, bias_b,
                       bias_h, sh.Hq, sh.Hkv, sh.Nq, sh.Nk, S, L, nrg, scale, scale * kLog2e,
                       xcd_pairs);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL, BIAS, 4>), dim3((unsigned)blocks),
                       dim3(256), 0, stream, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, ws_o, ws_ml, seqlens, (const uint16_t*)bias, bias_b,
                       bias_h, sh.Hq, sh.Hkv, sh.Nq, sh.Nk, S, L, nrg, scale, scale * kLog2e,
                       xcd_pairs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)rows), dim3(64), 0,
                     stream, (const float*)ws_o, (const float*)ws_ml, (uint16_t*)out, lse,
                     (int)rows, S, xcd_pairs, R);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_b(const void* q, const void* k, const void* v, void* out, float* lse,
                    float* ws_o, float* ws_ml, const int* seqlens, const void* bias, int bias_b,
                    int bias_h, const AttnShape& s, float scale, int S, hipStream_t stream) {
  return bias ? launch<D, CAUSAL, true>(q, k, v, out, lse, ws_o, ws_ml, seqlens, bias, bias_b,
                                        bias_h, s, scale, S, stream)
              : launch<D, CAUSAL, false>(q, k, v, out, lse, ws_o, ws_ml, seqlens, nullptr, 1, 1,
                                         s, scale, S, stream);
}

}  // namespace

hipError_t decode_scratch_address(hipStream_t stream, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> cached[kMaxDevices];
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = cached[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // the symbol's address on `dev`, taken with that device current (two threads racing here
    // both store the same address)
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = dev != cur ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (p == nullptr) return hipErrorInvalidSymbol;
    cached[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode_splitkv(const void* q, const void* k, const void* v, void* out,
                                 float* lse, float* ws_o, float* ws_ml, const int* seqlens,
                                 const void* bias, int bias_b, int bias_h, const AttnShape& s,
                                 float scale, bool causal, int n_splits, hipStream_t stream) {
  if (s.d == 128)
    return causal ? launch_b<128, true>(q, k, v, out, lse, ws_o, ws_ml, seqlens, bias, bias_b,
                                        bias_h, s, scale, n_splits, stream)
                  : launch_b<128, false>(q, k, v, out, lse, ws_o, ws_ml, seqlens, bias, bias_b,
                                         bias_h, s, scale, n_splits, stream);
  return causal ? launch_b<64, true>(q, k, v, out, lse, ws_o, ws_ml, seqlens, bias, bias_b, bias_h,
                                     s, scale, n_splits, stream)
                : launch_b<64, false>(q, k, v, out, lse, ws_o, ws_ml, seqlens, bias, bias_b,
                                      bias_h, s, scale, n_splits, stream);
}

}  // namespace fa
