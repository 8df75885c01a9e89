// C ABI of the attention library (declared in include/sdpa_fa2.h): argument validation, then
// the kernel launches.  Every check runs before anything is enqueued, so an error leaves all
// outputs untouched.  The library holds no state and never allocates or synchronises.
#include "sdpa_fa2.h"

#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace {

constexpr int kMaxSeq = 1 << 30;  // keeps every in-kernel index product inside 32/64-bit range
// Smallest non-zero scale accepted.  The kernels carry an additive bias in units of the unscaled
// dot product (bias / scale), so 1 / scale must stay finite with room to spare: with the floor,
// bias / scale is finite for every |bias| < 2^96.
constexpr float kMinScale = 0x1p-32f;

bool scale_ok(float scale) {
  return scale >= 0.f && isfinite(scale) && (scale == 0.f || scale >= kMinScale);
}

bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// elements of a [n0, n1, n2, n3] tensor; false on overflow
bool numel4(int n0, int n1, int n2, int n3, uint64_t* out) {
  uint64_t x = (uint64_t)n0;
  return mul_ok(x, (uint64_t)n1, &x) && mul_ok(x, (uint64_t)n2, &x) &&
         mul_ok(x, (uint64_t)n3, &x) && mul_ok(x, 4u, out);  // bytes of fp32 bound the bf16 case
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Shared checks.  Returns ATTN_OK and sets *empty when there is nothing to compute.
int check_common(const void* q, const void* k, const void* v, const void* out, const float* lse,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, bool* empty) {
  *empty = false;
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || d < 0) return ATTN_ERR_SHAPE;
  if (Nq >= kMaxSeq || Nk >= kMaxSeq) return ATTN_ERR_SHAPE;
  uint64_t tmp;
  if (!numel4(B, Hq, Nq, d, &tmp) || !numel4(B, Hkv, Nk, d, &tmp)) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  // one (batch, head) slice of K or V, plus one block of overrun, must be addressable by the
  // kernels' 32-bit buffer offsets
  if (((uint64_t)Nk + 128u) * (uint64_t)d * 2u > 0xffffffffull) return ATTN_ERR_SHAPE;
  if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0)) return ATTN_ERR_GQA;
  if (!scale_ok(scale)) return ATTN_ERR_SCALE;
  if ((uint64_t)B * (uint64_t)Hq * (uint64_t)Nq == 0) {
    *empty = true;
    return ATTN_OK;
  }
  if (q == nullptr || out == nullptr) return ATTN_ERR_NULL;
  if (Nk > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(lse, 4)) return ATTN_ERR_ALIGN;
  if (Nk > 0 && (!aligned(k, 16) || !aligned(v, 16))) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

float resolve_scale(float scale, int d) { return scale == 0.f ? 1.0f / sqrtf((float)d) : scale; }

int launch_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

// Checks of the optional extras: per-batch key lengths and the additive bias.
int check_extras(const int* seqlens_k, const void* bias, int bias_b, int bias_h, int B, int Hq,
                 int Nk) {
  if (seqlens_k != nullptr && !aligned(seqlens_k, 4)) return ATTN_ERR_ALIGN;
  if (bias == nullptr) return ATTN_OK;
  if (!(bias_b == 1 || bias_b == B) || !(bias_h == 1 || bias_h == Hq)) return ATTN_ERR_BIAS;
  if (Nk % 4 != 0) return ATTN_ERR_BIAS;
  if (!aligned(bias, 16)) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

// Prefill: launch-size check, then the kernel
int run_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
            const int* seqlens_k, const void* bias, int bias_b, int bias_h, int B, int Hq,
            int Hkv, int Nq, int Nk, int d, float scale, int causal, void* stream) {
  const long long blocks = (long long)B * Hq * ((Nq + 127) / 128);
  if (blocks > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  const fa::AttnShape s{B, Hq, Hkv, Nq, Nk, d};
  return launch_status(fa::launch_fwd_bf16(q, k, v, out, lse, seqlens_k, bias, bias_b, bias_h, s,
                                           resolve_scale(scale, d), causal != 0,
                                           (hipStream_t)stream));
}

// Split-KV decode after the common checks: split count, workspace, launch sizes
int run_decode(const void* q, const void* k, const void* v, void* out, float* lse,
               void* workspace, size_t workspace_bytes, const int* seqlens_k, const void* bias,
               int bias_b, int bias_h, int B, int Hq, int Hkv, int Nq, int Nk, int d,
               float scale, int causal, int n_splits, bool empty, void* stream) {
  if (n_splits < 1 || n_splits > (Nk > 1 ? Nk : 1)) return ATTN_ERR_SPLITS;
  if (empty) return ATTN_OK;
  const size_t need = attn_decode_workspace_bytes(B, Hq, Nq, d, n_splits);
  if (need == 0 || workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return ATTN_ERR_ALIGN;
  const long long R = (long long)(Hq / Hkv) * Nq;
  const long long blocks = (long long)B * Hkv * ((R + 15) / 16) * n_splits;
  const long long rows = (long long)B * Hq * Nq;
  if (blocks > 0x7fffffffLL || rows > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  float* ws_o = (float*)workspace;
  float* ws_ml = ws_o + (size_t)rows * n_splits * d;
  const fa::AttnShape s{B, Hq, Hkv, Nq, Nk, d};
  return launch_status(fa::launch_decode_splitkv(q, k, v, out, lse, ws_o, ws_ml, seqlens_k, bias,
                                                 bias_b, bias_h, s, resolve_scale(scale, d),
                                                 causal != 0, n_splits, (hipStream_t)stream));
}

constexpr int kRouteDecodeBelow = 32;  // query rows below which attn_forward takes split-KV

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
             int Hkv, int Nq, int Nk, int d, float scale, int causal, void* stream) {
  bool empty;
  int rc = check_common(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, scale, &empty);
  if (rc != ATTN_OK || empty) return rc;
  return run_fwd(q, k, v, out, lse, nullptr, nullptr, 1, 1, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                 stream);
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                const int* seqlens_k, const void* bias, int bias_b, int bias_h, int B, int Hq,
                int Hkv, int Nq, int Nk, int d, float scale, int causal, void* stream) {
  bool empty;
  int rc = check_common(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, scale, &empty);
  if (rc != ATTN_OK) return rc;
  rc = check_extras(seqlens_k, bias, bias_b, bias_h, B, Hq, Nk);
  if (rc != ATTN_OK || empty) return rc;
  return run_fwd(q, k, v, out, lse, seqlens_k, bias, bias_b, bias_h, B, Hq, Hkv, Nq, Nk, d, scale,
                 causal, stream);
}

int attn_fwd_f32(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                 int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, void* stream) {
  bool empty;
  int rc = check_common(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, scale, &empty);
  if (rc != ATTN_OK || empty) return rc;
  if (Hq > 65535 || B > 65535) return ATTN_ERR_SHAPE;
  const fa::AttnShape s{B, Hq, Hkv, Nq, Nk, d};
  return launch_status(fa::launch_fwd_f32((const float*)q, (const float*)k, (const float*)v,
                                          (float*)out, lse, s, resolve_scale(scale, d),
                                          causal != 0, (hipStream_t)stream));
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Nq, int d, int n_splits) {
  if (B < 0 || Hq < 0 || Nq < 0 || d < 0 || n_splits < 0) return 0;
  uint64_t x = (uint64_t)B;
  if (!mul_ok(x, (uint64_t)Hq, &x) || !mul_ok(x, (uint64_t)Nq, &x) ||
      !mul_ok(x, (uint64_t)n_splits, &x) || !mul_ok(x, (uint64_t)d + 2u, &x) ||
      !mul_ok(x, 4u, &x) || x > (uint64_t)SIZE_MAX)
    return 0;
  return (size_t)x;
}

int attn_decode_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                        void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq,
                        int Nk, int d, float scale, int causal, int n_splits, void* stream) {
  bool empty;
  int rc = check_common(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, scale, &empty);
  if (rc != ATTN_OK) return rc;
  return run_decode(q, k, v, out, lse, workspace, workspace_bytes, nullptr, nullptr, 1, 1, B, Hq,
                    Hkv, Nq, Nk, d, scale, causal, n_splits, empty, stream);
}

int attn_decode_splitkv_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, const int* seqlens_k,
                           const void* bias, int bias_b, int bias_h, int B, int Hq, int Hkv,
                           int Nq, int Nk, int d, float scale, int causal, int n_splits,
                           void* stream) {
  bool empty;
  int rc = check_common(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, scale, &empty);
  if (rc != ATTN_OK) return rc;
  rc = check_extras(seqlens_k, bias, bias_b, bias_h, B, Hq, Nk);
  if (rc != ATTN_OK) return rc;
  return run_decode(q, k, v, out, lse, workspace, workspace_bytes, seqlens_k, bias, bias_b,
                    bias_h, B, Hq, Hkv, Nq, Nk, d, scale, causal, n_splits, empty, stream);
}

int attn_decode_splitkv_noalloc(const void* q, const void* k, const void* v, void* out,
                                float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                float scale, int causal, int n_splits, void* stream) {
  bool empty;
  int rc = check_common(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, scale, &empty);
  if (rc != ATTN_OK) return rc;
  if (n_splits < 1 || n_splits > (Nk > 1 ? Nk : 1)) return ATTN_ERR_SPLITS;
  if (empty) return ATTN_OK;
  const size_t need = attn_decode_workspace_bytes(B, Hq, Nq, d, n_splits);
  if (need == 0 || need > fa::kDecodeScratchBytes) return ATTN_ERR_SCRATCH;
  void* scratch = nullptr;
  if (fa::decode_scratch_address((hipStream_t)stream, &scratch) != hipSuccess)
    return ATTN_ERR_LAUNCH;
  return run_decode(q, k, v, out, lse, scratch, fa::kDecodeScratchBytes, nullptr, nullptr, 1, 1,
                    B, Hq, Hkv, Nq, Nk, d, scale, causal, n_splits, false, stream);
}

int attn_decode_num_splits(int B, int Hq, int Hkv, int Nq, int Nk) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || Hq % Hkv != 0) return 1;
  // enough workgroups to give every compute unit a few (4 x 256), but at least 256 keys (two
  // 32-key blocks per wave) per split
  const long long per_split = (long long)B * Hkv * (((long long)(Hq / Hkv) * Nq + 15) / 16);
  const long long want = (1024 + per_split - 1) / per_split;
  const long long most = ((long long)Nk + 255) / 256;
  long long s = want < most ? want : most;
  if (s < 1) s = 1;
  if (s > 256) s = 256;
  return (int)s;
}

size_t attn_forward_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  if (Nq >= kRouteDecodeBelow) return 0;
  return attn_decode_workspace_bytes(B, Hq, Nq, d, attn_decode_num_splits(B, Hq, Hkv, Nq, Nk));
}

int attn_forward(const void* q, const void* k, const void* v, void* out, float* lse,
                 void* workspace, size_t workspace_bytes, const int* seqlens_k, const void* bias,
                 int bias_b, int bias_h, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, void* stream) {
  if (Nq >= kRouteDecodeBelow || Nk < 1)
    return attn_fwd_ex(q, k, v, out, lse, seqlens_k, bias, bias_b, bias_h, B, Hq, Hkv, Nq, Nk, d,
                       scale, causal, stream);
  return attn_decode_splitkv_ex(q, k, v, out, lse, workspace, workspace_bytes, seqlens_k, bias,
                                bias_b, bias_h, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                                attn_decode_num_splits(B, Hq, Hkv, Nq, Nk), stream);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Nq) {
  if (B < 0 || Hq < 0 || Nq < 0) return 0;
  uint64_t x = (uint64_t)B;
  if (!mul_ok(x, (uint64_t)Hq, &x) || !mul_ok(x, (uint64_t)Nq, &x) || !mul_ok(x, 8u, &x) ||
      x > (uint64_t)SIZE_MAX)
    return 0;
  return (size_t)x;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
             int causal, void* stream) {
  return attn_bwd_ex(q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace_bytes, nullptr,
                     nullptr, 1, 1, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream);
}

int attn_bwd_ex(const void* q, const void* k, const void* v, const void* out, const float* lse,
                const void* dout, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, const int* seqlens_k, const void* bias, int bias_b,
                int bias_h, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                int causal, void* stream) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || d < 0) return ATTN_ERR_SHAPE;
  if (Nq >= kMaxSeq || Nk >= kMaxSeq) return ATTN_ERR_SHAPE;
  uint64_t tmp;
  if (!numel4(B, Hq, Nq, d, &tmp) || !numel4(B, Hkv, Nk, d, &tmp)) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (((uint64_t)Nk + 128u) * (uint64_t)d * 2u > 0xffffffffull ||
      ((uint64_t)Nq + 128u) * (uint64_t)d * 2u > 0xffffffffull)
    return ATTN_ERR_SHAPE;
  if ((Hq > 0 || Hkv > 0) && (Hkv < 1 || Hq % Hkv != 0)) return ATTN_ERR_GQA;
  if (!scale_ok(scale)) return ATTN_ERR_SCALE;
  const bool has_q = (uint64_t)B * (uint64_t)Hq * (uint64_t)Nq > 0;
  const bool has_k = (uint64_t)B * (uint64_t)Hkv * (uint64_t)Nk > 0;
  if (!has_q && !has_k) return ATTN_OK;
  if (has_q && (q == nullptr || out == nullptr || lse == nullptr || dout == nullptr ||
                dq == nullptr))
    return ATTN_ERR_NULL;
  if (has_k && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
    return ATTN_ERR_NULL;
  if (has_q && (!aligned(q, 16) || !aligned(out, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
                !aligned(lse, 4)))
    return ATTN_ERR_ALIGN;
  if (has_k && (!aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) || !aligned(dv, 16)))
    return ATTN_ERR_ALIGN;
  if (has_q || has_k) {
    const int rc = check_extras(seqlens_k, bias, bias_b, bias_h, B, Hq, Nk);
    if (rc != ATTN_OK) return rc;
  }
  if (has_q) {
    const size_t need = attn_bwd_workspace_bytes(B, Hq, Nq);
    if (need == 0 || workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_ERR_ALIGN;
  }
  const long long gq = (long long)B * Hq * ((Nq + 127) / 128);
  const long long gk = (long long)B * Hkv * ((Nk + 127) / 128);
  if (gq > 0x7fffffffLL || gk > 0x7fffffffLL || (long long)B * Hq * Nq / 16 > 0x7fffffffLL)
    return ATTN_ERR_SHAPE;
  const fa::AttnShape s{B, Hq, Hkv, Nq, Nk, d};
  return launch_status(fa::launch_bwd_bf16(q, k, v, out, lse, dout, dq, dk, dv, (float*)workspace,
                                           seqlens_k, bias, bias_b, bias_h, s,
                                           resolve_scale(scale, d), causal != 0,
                                           (hipStream_t)stream));
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape: negative dimension or size overflow";
    case ATTN_ERR_HEADDIM: return "unsupported head dimension (must be 64 or 128)";
    case ATTN_ERR_GQA: return "Hq must be a positive multiple of Hkv";
    case ATTN_ERR_ALIGN: return "tensor base address is not suitably aligned";
    case ATTN_ERR_SCALE:
      return "scale must be 0 (selects 1/sqrt(d)) or a finite value >= 2^-32";
    case ATTN_ERR_SPLITS: return "n_splits must be in [1, max(Nk, 1)]";
    case ATTN_ERR_WORKSPACE: return "workspace is NULL or too small";
    case ATTN_ERR_LAUNCH: return "HIP kernel launch failed";
    case ATTN_ERR_BIAS:
      return "bias dims must be 1 or B (batch) and 1 or Hq (heads), and Nk a multiple of 4";
    case ATTN_ERR_SCRATCH:
      return "the split partials need more than the library's fixed 32 MiB decode scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
