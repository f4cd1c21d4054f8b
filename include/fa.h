/*
 * fa.h -- C ABI of libfa.so: exact tiled attention (FlashAttention-2 style) on MI355X.
 *
 * The operation.  For every sequence b and query head h,
 *     O = softmax(scale * Q K^T) V,        LSE_i = ln sum_j exp(scale * q_i . k_j),
 * where K, V are those of KV head h / (Hq / Hkv) (MQA/GQA: contiguous groups of query
 * heads share a KV head; Hq must be divisible by Hkv).  Sources: the FlashAttention
 * README (Dao-AILab/flash-attention, Chinese translation), "How to use FlashAttention":
 * the flash_attn_func docstring (definition, layouts, default scale 1/sqrt(headdim),
 * MQA/GQA rule); the flash_attn_with_kvcache docstring and changelog entry 2.1 (the
 * causal mask is aligned to the bottom-right corner: key j is kept for query i iff
 * j <= i + Lk - Lq, and a query row that keeps no key outputs zeros).  The LSE is
 * returned so that callers can drive the backward themselves or merge partial results
 * (kernels-community/flash-attn2 repository card, "Low-level ops"); it is the natural
 * logarithm, fp32, and +inf for a row that keeps no key.
 *
 * The score matrix never reaches device memory: scores are computed tile by tile with a
 * running (max, sum) softmax and discarded.
 *
 * Layouts (all tensors contiguous, innermost dimension D, base pointers 16-byte aligned):
 *   padded  (cu_seqlens_q == cu_seqlens_k == NULL):
 *     q, out, dout, dq : [B, Sq, Hq, D]        k, v, dk, dv : [B, Sk, Hkv, D]
 *     lse              : [B, Hq, Sq] fp32
 *   varlen  (both cu_seqlens given; int32 device arrays of length B+1, cu[0] = 0,
 *            non-decreasing; sequence b owns rows [cu[b], cu[b+1]) ):
 *     q, out, dout, dq : [total_q, Hq, D]      k, v, dk, dv : [total_k, Hkv, D]
 *     lse              : [Hq, total_q] fp32,   total_q = cu_seqlens_q[B]
 *     B = number of sequences; Sq / Sk = upper bounds of the per-sequence lengths (they
 *     size the launch grid).  total_q is read on the device; the host never syncs.
 *   dtype: FA_DTYPE_FP16 or FA_DTYPE_BF16 for every 16-bit tensor; accumulation is fp32.
 *   D: 64, 128 or 256.
 *
 * Ownership: the caller owns every buffer; the library allocates no device memory and
 * keeps no mutable global state except a thread-local last-error message.
 *
 * Errors: arguments are checked on the host before anything is launched; on error the
 * call returns a non-zero fa_status and writes nothing.  Work is enqueued on `stream`
 * (NULL = the default stream) and runs asynchronously; device faults surface at the
 * caller's next synchronisation.  No call synchronises the host or allocates memory,
 * so all of them may be captured into a HIP graph.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1, /* bad pointer, size, head ratio, scale or cu_seqlens pairing */
  FA_ERR_UNSUPPORTED = 2,      /* dtype or head dimension without a kernel */
  FA_ERR_WORKSPACE = 3,        /* backward workspace missing or too small */
  FA_ERR_HIP = 4               /* a HIP launch call failed (see fa_last_error) */
} fa_status;

typedef enum fa_dtype { FA_DTYPE_FP16 = 0, FA_DTYPE_BF16 = 1 } fa_dtype;

/*
 * Forward.  Writes out and lse (layouts above).  `scale` multiplies Q K^T before the
 * softmax (callers usually pass 1/sqrt(D)); it must be finite and >= 0.  `causal` != 0 applies
 * the bottom-right-aligned causal mask.  Rows of a varlen sequence beyond its length are
 * neither read nor written.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
           int B, int Sq, int Sk, int Hq, int Hkv, int D, float scale, int causal,
           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
           int dtype, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs: an fp32 dQ accumulator and an fp32 row
 * statistic (sum_d dO*O) for B*Sq rows of Hq heads (for varlen, B*Sq bounds total_q).
 * Returns 0 for invalid sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int Sq, int Hq, int D);

/*
 * Backward: given dout = dL/dO and the forward's own out and lse, writes
 * dq = dL/dQ, dk = dL/dK, dv = dL/dV (input dtype).  For GQA, dk/dv of a KV head sum
 * over its query heads.  The probabilities are recomputed from lse (no score matrix is
 * stored).  Other arguments as for fa_fwd.  `workspace` (16-byte aligned) must hold
 * fa_bwd_workspace_bytes(B, Sq, Hq, D) bytes; its contents on entry do not matter.
 * dq, dk, dv are fully overwritten (rows beyond a varlen sequence are not touched).
 * dq is accumulated with fp32 atomics, so the result may differ in the last bits from
 * run to run; the forward is bitwise deterministic.
 */
int fa_bwd(const void* dout, const void* q, const void* k, const void* v,
           const void* out, const float* lse, void* dq, void* dk, void* dv,
           int B, int Sq, int Sk, int Hq, int Hkv, int D, float scale, int causal,
           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
           int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Deterministic backward: same arguments, results and workspace as fa_bwd, but dQ is
 * formed by a separate pass over the key blocks of each query block instead of fp32
 * atomics, so dq, dk and dv are bitwise identical from run to run (the pages' README
 * offers a deterministic backward: changelog entry 2.4 and the `deterministic`
 * argument of the flash_attn_func docstring).  It recomputes the scores and dP once more,
 * so it is slower than fa_bwd.
 */
int fa_bwd_deterministic(const void* dout, const void* q, const void* k, const void* v,
                         const void* out, const float* lse, void* dq, void* dk, void* dv,
                         int B, int Sq, int Sk, int Hq, int Hkv, int D, float scale, int causal,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One stage of fa_bwd, for callers that schedule or time the stages themselves.
 * stage 1: preprocess -- per (row, head) Dsum = sum_d dout*out into the workspace and
 *          zeroing of the workspace's fp32 dQ accumulator (memory-bound);
 * stage 2: main loop -- dk, dv written, dQ (times scale) added into the accumulator;
 * stage 3: finalize -- dq = accumulator converted to the input dtype.
 * fa_bwd is stages 1, 2, 3 in this order on one stream; a stage reads what the earlier
 * stages left in the workspace.  Arguments, checks and errors as for fa_bwd; a stage
 * outside 1..3 returns FA_ERR_INVALID_ARGUMENT.
 */
int fa_bwd_stage(int stage, const void* dout, const void* q, const void* k, const void* v,
                 const void* out, const float* lse, void* dq, void* dk, void* dv,
                 int B, int Sq, int Sk, int Hq, int Hkv, int D, float scale, int causal,
                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                 int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* fa_status_string(int status);

/* Message describing the last error on the calling thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
