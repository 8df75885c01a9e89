// Device-side building blocks shared by the gfx950 attention kernels.
//
// Lane layouts used throughout (64-wide wavefront, measured on gfx950 with an in-bounds probe):
//   v_mfma_f32_32x32x16_bf16  D = A(32x16) * B(16x32) + C
//     A[i][k]: lane i + 32*(k/8), bf16 element k%8 of the 8-element operand
//     B[k][j]: lane j + 32*(k/8), element k%8
//     C[i][j]: lane j + 32*((i/4)%2), fp32 register 4*(i/8) + i%4   (16 registers)
//   v_permlane32_swap(x, x) returns {x[l%32], x[l%32 + 32]} in every lane l.
//   ds_read_b64_tr_b16: within each 16-lane group, output lane i element j is element i%4 of the
//     four b16 values that source lane 4*j + i/4 of the group addresses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef bf16x4 __attribute__((address_space(3))) lds_bf16x4;

constexpr float kLog2e = 1.4426950408889634f;

// fp32 accumulate of a 16x16x32 bf16 product (layout as above with 16-lane groups:
// A[i][k] in lane i + 16*(k/8), element k%8; C[i][j] in lane j + 16*(i/4), register i%4).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 accumulate of a 32x32x16 bf16 product; operands travel as raw 32-bit words.
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two fp32 values -> one word of two bf16 (round to nearest even), `lo` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// 2^x on the transcendental unit (v_exp_f32); exact 0 for -inf.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of x over the lane pair (l, l ^ 32); both lanes get the identical result.
__device__ __forceinline__ float pair32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing 8-byte LDS read (see the layout note above).
__device__ __forceinline__ bf16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

// The 8-element MFMA operand made of two transposing reads (first read -> elements 0..3).
__device__ __forceinline__ bf16x8 lds_read_tr16_pair(const uint16_t* p0, const uint16_t* p1) {
  return __builtin_shufflevector(lds_read_tr16(p0), lds_read_tr16(p1), 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Lazy rescaling of the online softmax: the running max m that exponents are taken against is
// only moved when a block's max exceeds it by more than this many powers of two, so the
// probabilities stay below 2^kLazyLog2 and the accumulator is rarely rescaled.  O and l always
// share the same reference max, so the final O / l is unchanged.
constexpr float kLazyLog2 = 8.0f;
// Largest block-to-block rise of the max (log2 units) that a rescale may absorb in registers
// from probabilities already computed against the old reference: 2^120 is still finite in fp32
// and bf16.
constexpr float kShiftMax = 120.0f;

// Buffer resource covering `bytes` bytes from `base` (raw addressing, no stride).  Buffer loads
// through it read zero past the end, which is how K/V rows beyond the sequence are filled.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16 bytes per lane from `rsrc` at byte offset voff + soff straight into LDS: lane i's bytes
// land at `lds_base` + 16 i (`lds_base` and `soff` must be the same for the whole wave).  Both
// offsets take part in the range check.  The instruction's immediate offset field is left at
// zero on purpose: it would also move the LDS destination (measured on gfx950).
__device__ __forceinline__ void load_lds_16(__amdgpu_buffer_rsrc_t rsrc, void* lds_base,
                                            uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)lds_base, 16, (int)voff, (int)soff, 0, 0);
}

// The same with 4 bytes per lane: lane i's bytes land at `lds_base` + 4 i.
__device__ __forceinline__ void load_lds_4(__amdgpu_buffer_rsrc_t rsrc, void* lds_base,
                                           uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)lds_base, 4, (int)voff, 0, 0, 0);
}

// 16 bytes per lane from `rsrc` at byte offset voff + soff into registers (zero past the end),
// marked non-temporal (cache-policy bit 1): for data read exactly once, such as the keys and
// values a decode split streams, this measured ~15% faster than the default policy on gfx950.
__device__ __forceinline__ u32x4 load_16_stream(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                                uint32_t soff) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)voff, (int)soff, 2));
}

// Wait until this wave's outstanding vector-memory loads (including LDS-direct ones) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 64 lanes of the wave vote: true when the predicate holds in any active lane.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }
__device__ __forceinline__ bool wave_all(bool p) { return !wave_any(!p); }

}  // namespace fa
