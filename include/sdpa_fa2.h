/*
 * sdpa_fa2.h -- C ABI of the MI355X (gfx950) fused scaled-dot-product attention library.
 *
 * The library computes O = softmax(scale * Q Kᵀ + causal mask) V and the per-row logsumexp,
 * the naive five-step attention of "PyTorch 어텐션 프로파일링 Flash, cuDNN, Math 백엔드 완벽 비교"
 * (section 1: matmul, scale, masked_fill(-inf), softmax, matmul), without ever writing the
 * [seq, seq] score matrix to memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory:  every tensor pointer is a DEVICE pointer (HIP device memory, or memory the device can
 *          address).  The caller allocates and frees every buffer, including the decode
 *          workspace; the library never allocates, frees or synchronises, and keeps no state
 *          beyond its loaded code objects (which include the fixed scratch array of
 *          attn_decode_splitkv_noalloc) and that entry point's cached per-device address of it.
 * Layout:  contiguous row-major tensors in the native [batch, heads, seq, head_dim] order
 *          ("BNSH"), head_dim fastest:  q, out: [B, Hq, Nq, d];  k, v: [B, Hkv, Nk, d];
 *          lse: [B, Hq, Nq] float32.  No transposes are taken or required.
 * GQA:     Hq must be a multiple of Hkv; query head hq reads K/V head hq / (Hq / Hkv)
 *          (K/V heads broadcast to groups of query heads, as in the FlashAttention-2 notes'
 *          grouped-query example, "FlashAttention-2: Faster Attention with Better Parallelism
 *          and Work Partitioning", code example).
 * Scale:   scores are multiplied by `scale` before masking; scale == 0 selects 1/sqrt(d) (the
 *          default of the WebGPU decode program, "[onnxruntime] WebGPU FlashAttention 최적화",
 *          section 2).  A negative or non-finite scale, or a positive one below 2^-32, is
 *          rejected (the kernels carry a bias as bias / scale, which must stay finite).
 * Causal:  when `causal` is non-zero, key j is visible to query i iff j <= i + (Nk - Nq), i.e. the
 *          mask is aligned to the end of the keys; with Nq == Nk it is the usual lower triangle.
 *          A query row with no visible key gets out = 0 and lse = -inf.
 * LSE:     lse[b,h,i] = ln sum_j exp(scale * q_i . k_j) over visible j (natural log), float32.
 *          `lse` may be NULL, in which case it is not written.
 * Shapes:  every dimension must be >= 0; d must be 64 or 128; one K/V head slice must stay below
 *          4 GiB ((Nk + 128) * d * 2 < 2^32, i.e. Nk < 16,777,088 at d = 128) and Nq, Nk < 2^30.
 *          An empty problem (B*Hq*Nq == 0)
 *          returns ATTN_OK without launching anything.  Nk == 0 is allowed (all rows empty).
 * Pointers: q/out must be non-NULL when B*Hq*Nq > 0, k/v when additionally Nk > 0; q, k, v, out
 *          and the workspace must be 16-byte aligned, lse 4-byte aligned.
 * Streams: `stream` is a hipStream_t (NULL = the default stream).  Every call only enqueues work
 *          on that stream and returns; outputs are valid once the stream reaches that point.
 * Errors:  every check runs before anything is enqueued; on error nothing is written and a
 *          negative ATTN_ERR_* code is returned.  ATTN_ERR_LAUNCH reports a HIP launch failure.
 *          Kernels have no other failure mode; NaN/Inf inputs propagate into the outputs.
 */
#ifndef SDPA_FA2_H
#define SDPA_FA2_H

#include <stddef.h>

#if defined(__GNUC__)
#define SDPA_FA2_API __attribute__((visibility("default")))
#else
#define SDPA_FA2_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,      /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,     /* a negative dimension, a size that overflows, or a too-long K/V */
  ATTN_ERR_HEADDIM = -3,   /* d is not 64 or 128 */
  ATTN_ERR_GQA = -4,       /* Hkv < 1 while Hq > 0, or Hq % Hkv != 0 */
  ATTN_ERR_ALIGN = -5,     /* a tensor base address is not suitably aligned */
  ATTN_ERR_SCALE = -6,     /* scale is negative, NaN, infinite, or in (0, 2^-32) */
  ATTN_ERR_SPLITS = -7,    /* n_splits < 1 or n_splits > max(Nk, 1) */
  ATTN_ERR_WORKSPACE = -8, /* workspace NULL or smaller than its *_workspace_bytes() size */
  ATTN_ERR_LAUNCH = -9,    /* the HIP runtime rejected a kernel launch */
  ATTN_ERR_BIAS = -10,     /* bias_b not 1 or B, bias_h not 1 or Hq, or Nk % 4 != 0 with a bias */
  ATTN_ERR_SCRATCH = -11   /* attn_decode_splitkv_noalloc: the partials exceed its fixed scratch */
};

/*
 * attn_fwd -- fused attention forward (prefill), bfloat16 in and out, fp32 accumulation.
 *
 * Implements the FlashAttention-2 forward of "FlashAttention-2: Faster Attention with Better
 * Parallelism and Work Partitioning" (section "방법론 / 알고리즘 개요": Q block outer loop, K/V
 * block inner loop, running max and sum, one final 1/l; section "인과적 마스킹 최적화": blocks
 * above the diagonal skipped; section "개선 2": parallel over batch x heads x Q blocks).
 *
 *   q   [B, Hq, Nq, d]  bf16 (read)        k, v [B, Hkv, Nk, d] bf16 (read)
 *   out [B, Hq, Nq, d]  bf16 (written, round-to-nearest-even from fp32)
 *   lse [B, Hq, Nq]     fp32 (written unless NULL)
 */
SDPA_FA2_API int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int Hq, int Hkv, int Nq, int Nk, int d,
             float scale, int causal, void* stream);

/*
 * attn_fwd_f32 -- the same operation with float32 q, k, v and out (fp32 arithmetic throughout).
 * Same arguments, layouts and errors as attn_fwd; the tensors hold float32 instead of bf16.
 */
SDPA_FA2_API int attn_fwd_f32(const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, void* stream);

/*
 * attn_decode_workspace_bytes -- bytes of device workspace attn_decode_splitkv needs:
 *   B*Hq*Nq*n_splits*(d + 2)*4: one fp32 partial output row of d values plus the (local max,
 *   local sum) pair per query row and split, the out_split_vx / metadata outputs of the fused
 *   decode program of "[onnxruntime] WebGPU FlashAttention 최적화: 커널 퓨전과 가변 시퀀스 길이
 *   지원으로 성능 극대화" (section 1).  The caller owns this memory, as a library workspace is
 *   the caller's memory in "3.3 cuDNN II — 그래프 융합 API·휴리스틱" (section 3.3.2, the workspace
 *   trade-off).
 *   Host-only arithmetic, no device access.  Returns 0 for negative arguments or when the size
 *   overflows size_t.
 */
SDPA_FA2_API size_t attn_decode_workspace_bytes(int B, int Hq, int Nq, int d, int n_splits);

/*
 * attn_decode_splitkv -- split-KV attention for few query rows against a long K/V.
 *
 * Two launches on `stream`, following the fused decode program and its reduce step of
 * "[onnxruntime] WebGPU FlashAttention 최적화: 커널 퓨전과 가변 시퀀스 길이 지원으로 성능 극대화"
 * (section 1, kernel fusion; section 2, several query rows per workgroup):
 *   1. split kernel: for each (batch, KV head, split) the keys [s*L, min((s+1)*L, Nk)),
 *      L = ceil(Nk / n_splits), are read once for all Hq/Hkv * Nq query rows of that KV head;
 *      each row gets a locally normalised partial output O_s plus metadata (m_s, l_s):
 *      m_s = max of the scaled visible scores in the split, l_s = sum exp(score - m_s).
 *   2. combine kernel: M = max_s m_s, w_s = l_s exp(m_s - M), out = sum_s w_s O_s / sum_s w_s,
 *      lse = M + ln sum_s w_s.
 * Same q/k/v/out/lse conventions as attn_fwd (bf16 tensors).  The causal mask is aligned to the
 * end of the keys (the usual decode case: the Nq new tokens are the last Nq positions).
 *
 * workspace: device memory of at least attn_decode_workspace_bytes(B, Hq, Nq, d, n_splits)
 *   bytes, owned by the caller, fully overwritten by each call:
 *     ws_O  float32 [B, Hq, Nq, n_splits, d]   (locally normalised partial outputs)
 *     ws_ml float32 [B, Hq, Nq, n_splits, 2]   ((m_s, l_s); empty split: (-inf, 0))
 *   stored back to back, ws_O first.  Calls that share a workspace must be stream ordered.
 */
SDPA_FA2_API int attn_decode_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                        void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d,
                        float scale, int causal, int n_splits, void* stream);

/*
 * attn_decode_splitkv_noalloc -- attn_decode_splitkv for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments, layouts, kernels and results as attn_decode_splitkv (bit-identical), without
 * the workspace pair: the split partials go to a fixed 32 MiB array of device memory inside the
 * library instead (one per GPU, held from the library's first use of that GPU until the process
 * ends).  The call allocates and frees nothing: the array's device address is looked up once per
 * device (on the first call whose stream is on that device) and cached.
 *   Limit: attn_decode_workspace_bytes(B, Hq, Nq, d, n_splits) <= 33,554,432 bytes, else
 *   ATTN_ERR_SCRATCH and nothing is enqueued (e.g. B=8, Hq=32, Nq=4, d=128, 16 splits needs
 *   8,519,680 bytes).
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents (each call
 * overwrites every partial it reads, so nothing needs clearing first).  Calls that may overlap on
 * one GPU -- on different streams without ordering, or from several threads -- race on the array
 * and must not be issued; calls on one stream are ordered.  ATTN_ERR_LAUNCH also reports a failed
 * address lookup.
 */
SDPA_FA2_API int attn_decode_splitkv_noalloc(const void* q, const void* k, const void* v,
                                             void* out, float* lse, int B, int Hq, int Hkv,
                                             int Nq, int Nk, int d, float scale, int causal,
                                             int n_splits, void* stream);

/*
 * Extras of the *_ex entry points and of attn_forward (all optional: NULL means "none").
 *
 * seqlens_k  DEVICE pointer to int32 [B], 4-byte aligned, or NULL.  seqlens_k[b] is the number of
 *            valid keys of batch element b: only K/V rows 0 .. seqlens_k[b]-1 exist for it, and
 *            the causal mask is aligned to the end of those keys (key j visible to query i iff
 *            j <= i + seqlens_k[b] - Nq).  Nk is then the capacity (the seq dimension of k and
 *            v).  Values are read on the device and clamped to [0, Nk]; a batch element with no
 *            key gets out = 0 and lse = -inf.  These are the per-batch KV lengths that the
 *            onnxruntime WebGPU page's decode path reads on the GPU ("[onnxruntime] WebGPU
 *            FlashAttention 최적화: 커널 퓨전과 가변 시퀀스 길이 지원으로 성능 극대화", the varlen part
 *            of its title and its seqlens_k inputs).  Split-KV chunks stay those of the capacity
 *            Nk, clipped to each element's length.
 * bias       DEVICE pointer to bf16 [bias_b, bias_h, Nq, Nk], contiguous, 16-byte aligned, or
 *            NULL; bias_b is 1 or B and bias_h is 1 or Hq (a size-1 dimension is broadcast), and
 *            Nk must be a multiple of 4.  The bias is added to the scaled scores before the mask
 *            (s = scale * q.k + bias), the attention bias of the same page's fused decode program
 *            (section 1); a -inf entry masks its key.  With seqlens_k, bias columns at or past
 *            seqlens_k[b] are never used (their values do not matter).  bias_b / bias_h are ignored when bias is NULL.
 *
 * Errors added by the extras: ATTN_ERR_BIAS (dims or Nk % 4) and ATTN_ERR_ALIGN (alignment).
 */

/*
 * attn_fwd_ex -- attn_fwd with per-batch key lengths and an additive bias (see above).  With
 * seqlens_k == NULL and bias == NULL it is exactly attn_fwd.  bfloat16 tensors only.
 */
SDPA_FA2_API int attn_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                const int* seqlens_k, const void* bias, int bias_b, int bias_h,
                int B, int Hq, int Hkv, int Nq, int Nk, int d,
                float scale, int causal, void* stream);

/*
 * attn_decode_splitkv_ex -- attn_decode_splitkv with per-batch key lengths and an additive bias
 * (see above).  Same workspace contract as attn_decode_splitkv.
 */
SDPA_FA2_API int attn_decode_splitkv_ex(const void* q, const void* k, const void* v, void* out,
                           float* lse, void* workspace, size_t workspace_bytes,
                           const int* seqlens_k, const void* bias, int bias_b, int bias_h,
                           int B, int Hq, int Hkv, int Nq, int Nk, int d,
                           float scale, int causal, int n_splits, void* stream);

/*
 * attn_decode_num_splits -- the split count attn_forward uses for split-KV: enough workgroups
 * (B * Hkv * ceil(Hq/Hkv * Nq / 16) per split) for about 1024 in all, but no split shorter than
 * 256 keys, and at most 256 splits.  Returns 1 for degenerate or invalid arguments.
 */
SDPA_FA2_API int attn_decode_num_splits(int B, int Hq, int Hkv, int Nq, int Nk);

/*
 * attn_forward_workspace_bytes -- workspace attn_forward needs for these sizes: 0 when it takes
 * the prefill kernel (Nq >= 32), else attn_decode_workspace_bytes with attn_decode_num_splits.
 */
SDPA_FA2_API size_t attn_forward_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d);

/*
 * attn_forward -- one entry for any query length, with the routing rule of the onnxruntime
 * WebGPU page (section "3. 경로 라우팅 최적화": split-reduce below 32 query rows, the prefill
 * program otherwise):
 *   Nq <  32 (and Nk >= 1): attn_decode_splitkv_ex with attn_decode_num_splits splits; the
 *            workspace must hold attn_forward_workspace_bytes bytes.
 *   Nq >= 32 (or Nk == 0):  attn_fwd_ex; workspace is not used and may be NULL.
 * Arguments and errors as for those two entry points.
 */
SDPA_FA2_API int attn_forward(const void* q, const void* k, const void* v, void* out, float* lse,
                 void* workspace, size_t workspace_bytes,
                 const int* seqlens_k, const void* bias, int bias_b, int bias_h,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, void* stream);

/*
 * attn_bwd_workspace_bytes -- bytes of device workspace attn_bwd needs: B*Hq*Nq*8 (two floats
 * per query row).  Returns 0 for invalid (negative) arguments.
 */
SDPA_FA2_API size_t attn_bwd_workspace_bytes(int B, int Hq, int Nq);

/*
 * attn_bwd -- gradients of the attention forward (attn_fwd), bfloat16 in and out, fp32
 * accumulation, head dimension 64 or 128.  Not on the pages (they only report the backward's
 * speed): the gradients of L = sum(dout * out) by the chain rule through the forward's steps,
 *   D_i = sum_d dout_id out_id,  P = exp(scale * q.k - lse) (masked positions 0),
 *   dv = P^T dout,  dS = P * (dout v^T - D),  dq = scale * dS k,  dk = scale * dS^T q,
 * with dk, dv summed over the Hq/Hkv query heads that share a K/V head.
 *
 *   q, dq [B, Hq, Nq, d]; k, v, dk, dv [B, Hkv, Nk, d]  bf16 (dq, dk, dv written)
 *   out, dout [B, Hq, Nq, d] bf16: the forward output and the gradient of the loss w.r.t. it
 *   lse [B, Hq, Nq] fp32: the forward's logsumexp (required; -inf rows get zero gradients)
 *   workspace: at least attn_bwd_workspace_bytes(B, Hq, Nq) bytes of device memory owned by the
 *     caller: fp32 -D [B, Hq, Nq], then -lse / scale [B, Hq, Nq] (-inf for -inf rows), both
 *     overwritten; calls that share it must be stream ordered.
 * scale and causal must be those of the forward call.  Keys that no query sees get dk = dv = 0;
 * with Nq == 0 and Nk > 0 the call writes zeros to dk and dv.  Errors as for attn_fwd (Nq, like
 * Nk, must keep one head slice below 4 GiB).
 */
SDPA_FA2_API int attn_bwd(const void* q, const void* k, const void* v, const void* out,
             const float* lse, const void* dout, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes,
             int B, int Hq, int Hkv, int Nq, int Nk, int d,
             float scale, int causal, void* stream);

/*
 * attn_bwd_ex -- attn_bwd for a forward that took the extras (attn_fwd_ex): per-batch key
 * lengths and an additive bias, with the meanings and checks of the extras above (NULL for
 * either means none; both NULL makes the call attn_bwd).  With seqlens_k element b has only its
 * first seqlens_k[b] keys, with the causal mask aligned to their end, and the K/V rows past them,
 * which take no part in the forward, get dk = dv = 0 (every row of dk and dv up to Nk is
 * written).  The bias enters P exactly as in the forward and is a constant: no gradient is
 * computed for it.  Other arguments and errors as for attn_bwd; out and lse must come from the
 * forward with the same extras.
 */
SDPA_FA2_API int attn_bwd_ex(const void* q, const void* k, const void* v, const void* out,
                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                void* workspace, size_t workspace_bytes, const int* seqlens_k,
                const void* bias, int bias_b, int bias_h,
                int B, int Hq, int Hkv, int Nq, int Nk, int d,
                float scale, int causal, void* stream);

/*
 * attn_status_string -- a static, NUL-terminated English description of a status code returned
 * by the entry points above (the counterpart of the Status that the onnxruntime WebGPU page's
 * host functions return, "[onnxruntime] WebGPU FlashAttention 최적화: 커널 퓨전과 가변 시퀀스
 * 길이 지원으로 성능 극대화", the ComputeFlashAttentionDecodeQKV code under section 3).  Host-only; never NULL; unknown
 * codes give "unknown status".  The string is owned by the library and must not be freed.
 */
SDPA_FA2_API const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_FA2_H */
