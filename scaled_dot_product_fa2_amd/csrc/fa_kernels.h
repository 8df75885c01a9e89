// Host-side launchers of the gfx950 kernels (internal to the library; the public ABI is
// include/sdpa_fa2.h).  Arguments are assumed validated by the C-ABI layer: non-empty shapes,
// d in {64, 128}, Hq % Hkv == 0, aligned pointers, finite positive scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct AttnShape {
  int B, Hq, Hkv, Nq, Nk, d;
};

// Prefill forward, bf16 tensors (fwd_bf16.hip).  seqlens: NULL or device int32 [B] key counts;
// bias: NULL or bf16 [bias_b, bias_h, Nq, Nk] (Nk % 4 == 0, 16-byte aligned base).
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                           const int* seqlens, const void* bias, int bias_b, int bias_h,
                           const AttnShape& s, float scale, bool causal, hipStream_t stream);

// Prefill forward, fp32 tensors (fwd_f32.hip).
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* out,
                          float* lse, const AttnShape& s, float scale, bool causal,
                          hipStream_t stream);

// Split-KV decode: split kernel then combine kernel on `stream` (decode.hip).
// ws_o: fp32 [B, Hq, Nq, n_splits, d]; ws_ml: fp32 [B, Hq, Nq, n_splits, 2]; seqlens and bias as
// for the prefill.
hipError_t launch_decode_splitkv(const void* q, const void* k, const void* v, void* out,
                                 float* lse, float* ws_o, float* ws_ml, const int* seqlens,
                                 const void* bias, int bias_b, int bias_h, const AttnShape& s,
                                 float scale, bool causal, int n_splits, hipStream_t stream);

// Bytes of the fixed device scratch array behind attn_decode_splitkv_noalloc (decode.hip).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;

// Device address of that array on the device of `stream` (the current device for the NULL
// stream), looked up once per device with hipGetSymbolAddress and cached.  Allocates nothing.
hipError_t decode_scratch_address(hipStream_t stream, void** ptr);

// Backward (bwd_bf16.hip), head dim 64 or 128: D = rowsum(dout * out) into ws_d (fp32 [B, Hq, Nq]),
// then dk/dv and dq; lse is the forward's natural-log logsumexp.  seqlens (device int32 [B], or
// nullptr) limits batch element b to its first seqlens[b] keys, and bias (bf16 [bias_b, bias_h,
// Nq, Nk], or nullptr) is added to the scores, both as in the forward.
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* ws_d, const int* seqlens, const void* bias, int bias_b,
                           int bias_h, const AttnShape& s, float scale, bool causal,
                           hipStream_t stream);

}  // namespace fa
