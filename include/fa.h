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
 *   D (head dimension): any multiple of 8 from 8 to 256.  The kernels are built for tile
 *   widths 64, 128 and 256; another D runs in the next wider one, its padding never read
 *   into a result and never written (flash_attn_func docstring and README "Installation
 *   and features": head dimensions up to 256).
 *
 * Ownership: the caller owns every buffer; the library allocates no device memory and
 * keeps no mutable global state except a thread-local last-error message and, on each
 * device, two static device arrays of its own: the 4-byte flag of the device-side checks
 * described next (zero unless FA_DEBUG_CHECKS=1 found an error) and the scratch array of
 * fa_fwd_kvcache_noalloc.
 *
 * Errors: arguments are checked on the host before anything is launched; on error the
 * call returns a non-zero fa_status and writes nothing.  Work is enqueued on `stream`
 * (NULL = the default stream) and runs asynchronously; device faults surface at the
 * caller's next synchronisation.  No call synchronises the host or allocates memory,
 * so all of them may be captured into a HIP graph.
 *
 * Device-side preconditions -- values the host cannot read without a synchronisation:
 * cu_seqlens_q / cu_seqlens_k start at 0, never decrease, and no sequence is longer than
 * Sq / Sk (so total_q <= B * Sq, the rows a backward workspace holds); the indices,
 * lengths and block-table entries of fa_fwd_kvcache address existing cache entries.  They
 * are the caller's contract.  With FA_DEBUG_CHECKS=1 in the environment every call that
 * depends on them first checks them on the device, and if one fails every kernel on that
 * device does nothing until fa_debug_status() reports the failure (see there).
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
 * Forward with a sliding window and/or ALiBi (flash_attn_func docstring, "How to use
 * FlashAttention": window_size and alibi_slopes arguments; changelog entries 2.3 and
 * 2.4).  Query i keeps key j iff
 *     i + Lk - Lq - window_left <= j <= i + Lk - Lq + window_right
 * (-1 = that side unbounded) and, if causal, j <= i + Lk - Lq, per sequence.  With
 * alibi_slopes (NULL: none; fp32 device array, slope of (b, h) at
 * alibi_slopes[b * alibi_batch_stride + h], stride 0 or Hq) the bias
 * -slope * |i + Lk - Lq - j| is added to the scaled score; the LSE is that of the biased
 * scores.  fa_fwd(...) is fa_fwd_ex(..., -1, -1, NULL, 0, ...).  Other arguments, layouts
 * and errors as for fa_fwd; window sizes below -1 or another stride are rejected.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse,
              int B, int Sq, int Sk, int Hq, int Hkv, int D, float scale, int causal,
              int window_left, int window_right, const float* alibi_slopes, int alibi_batch_stride,
              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
              int dtype, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs: an fp32 dQ accumulator and two fp32 row
 * statistics (sum_d dO*O and LSE*log2(e)) for B*Sq rows of Hq heads (for varlen, B*Sq
 * bounds total_q), plus 256 bytes for the work queue of the main loop.  Returns 0 for invalid sizes.
 * A workspace serves one backward at a time: calls that share one must not overlap.
 */
size_t fa_bwd_workspace_bytes(int B, int Sq, int Hq, int D);

/* Largest stored-dS area fa_bwd_ds_workspace_bytes offers (32 GiB). */
#define FA_BWD_DS_MAX_BYTES ((size_t)32 << 30)

/*
 * Extra workspace bytes, beyond fa_bwd_workspace_bytes(B, Sq, Hq, D), of the backward's
 * stored-dS route: the main loop writes dS / scale (the input dtype, rounded exactly as
 * the dQ product would take it) for every query step and key block it visits, and a
 * second, memory-bound pass forms dQ = scale dS K from them, with no atomics and no second
 * computation of S and dP.  The area is B * Hq * ceil(Sq / 32) * ceil(Sk / KB) tiles of
 * 32 * KB 16-bit values, KB = 256 keys for D <= 128 and 128 above (Sq, Sk the padded or
 * maximum lengths); only the tiles a mask keeps are written and read.  Returns 0 for
 * invalid sizes and when the area would exceed FA_BWD_DS_MAX_BYTES (the route is then not
 * available).
 */
size_t fa_bwd_ds_workspace_bytes(int B, int Sq, int Sk, int Hq, int D);

/*
 * Backward: given dout = dL/dO and the forward's own out and lse, writes
 * dq = dL/dQ, dk = dL/dK, dv = dL/dV (input dtype).  The method is the recompute-from-LSE
 * backward of the release notes "v1.4 - FlashAttention Fork" (section 4.1: the stored LSE,
 * times log2(e), is the exp2 offset that recovers P = exp(scale * q.k - LSE) tile by tile)
 * with the gradient of the definition above: dV = P^T dO, dP = dO V^T, Dsum_i =
 * sum_d dO_id O_id, dS = P * (dP - Dsum), dQ = scale dS K, dK = scale dS^T Q; the
 * kernels-community/flash-attn2 repository card ("Low-level ops") describes the same
 * split: a forward that returns (out, LSE) and a backward the caller drives with them.
 * For GQA, dk/dv of a KV head sum over its query heads.  The probabilities are recomputed from lse (no score matrix is
 * stored).  Other arguments as for fa_fwd.  `workspace` (16-byte aligned) must hold
 * fa_bwd_workspace_bytes(B, Sq, Hq, D) bytes; its contents on entry do not matter.
 * dq, dk, dv are fully overwritten (rows beyond a varlen sequence are not touched).
 * Route: for D > 64, when fa_bwd_ds_workspace_bytes(B, Sq, Sk, Hq, D) is nonzero and the
 * workspace holds both sizes, dQ is formed from the stored dS (the fastest route there, and
 * bitwise repeatable; the dS area follows the first fa_bwd_workspace_bytes bytes, rounded
 * up to 256).  Otherwise, for D <= 128, dq is accumulated with fp32 atomics, so the result
 * may differ in the last bits from run to run (for D <= 64 this route is the faster one),
 * and for D > 128 fa_bwd runs the recompute scheme of fa_bwd_deterministic.  The forward is
 * bitwise deterministic.
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
 * argument of the flash_attn_func docstring).  With a workspace large enough for the
 * stored-dS route (see fa_bwd) it runs that route at every D; otherwise it recomputes the
 * scores and dP once more in the dQ pass, which for D <= 128 is slower than fa_bwd's
 * atomic route.
 */
int fa_bwd_deterministic(const void* dout, const void* q, const void* k, const void* v,
                         const void* out, const float* lse, void* dq, void* dk, void* dv,
                         int B, int Sq, int Sk, int Hq, int Hkv, int D, float scale, int causal,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward with a sliding window and/or ALiBi, the counterpart of fa_fwd_ex (same mask and
 * bias arguments; out and lse must come from fa_fwd_ex with the same ones).  The bias does
 * not depend on q, k or v, so the gradient formulas are unchanged; masked pairs get zero
 * gradient.  deterministic != 0 selects the fa_bwd_deterministic scheme.  Workspace and
 * errors as for fa_bwd.
 */
int fa_bwd_ex(const void* dout, const void* q, const void* k, const void* v,
              const void* out, const float* lse, void* dq, void* dk, void* dv,
              int B, int Sq, int Sk, int Hq, int Hkv, int D, float scale, int causal,
              int window_left, int window_right, const float* alibi_slopes, int alibi_batch_stride,
              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
              int dtype, int deterministic, void* workspace, size_t workspace_bytes,
              hipStream_t stream);

/*
 * One stage of fa_bwd, for callers that schedule or time the stages themselves.
 * stage 1: preprocess -- per (row, head) -Dsum = -sum_d dout*out and LSE*log2(e) into the
 *          workspace, and zeroing of the workspace's fp32 dQ accumulator (memory-bound);
 * stage 2: main loop -- dk, dv written, dQ / scale added into the accumulator
 *          (its key-block queue is emptied by stage 1 and again at its own end, so it
 *          may be repeated on its own after a complete stage 1 or stage 2);
 * stage 3: finalize -- dq = scale * accumulator, in the input dtype;
 * stage 4: main loop of the stored-dS route -- dk, dv written, dS / scale stored in the
 *          workspace's dS area (needs the workspace of that route, see fa_bwd);
 * stage 5: dQ of the stored-dS route -- dq = scale dS K from the stored dS.
 * Stages 1, 4, 5 in this order are fa_bwd's stored-dS route; stages 1, 2, 3 its atomic
 * route (for D > 128 without the dS area fa_bwd takes the recompute route of
 * fa_bwd_deterministic instead; stages 1, 2, 3 still compute the same gradients there,
 * with atomics).  A stage reads what the earlier stages left in the workspace.  Arguments,
 * checks and errors as for fa_bwd; a stage outside 1..5 returns FA_ERR_INVALID_ARGUMENT,
 * and stage 4 or 5 without the dS area FA_ERR_WORKSPACE.
 */
int fa_bwd_stage(int stage, const void* dout, const void* q, const void* k, const void* v,
                 const void* out, const float* lse, void* dq, void* dk, void* dv,
                 int B, int Sq, int Sk, int Hq, int Hkv, int D, float scale, int causal,
                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                 int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Attention of a few new query rows against a read-only KV cache (incremental decoding).
 * Sources: the flash_attn_with_kvcache docstring in "How to use FlashAttention" (cache
 * layouts, cache_seqlens, cache_batch_idx, block_table, causal and window alignment,
 * ALiBi) and changelog entry 2.2 (split the cache over workgroups and merge the partial
 * results in a separate kernel) of the FlashAttention README.  Appending new keys to the
 * cache and rotary embeddings are not part of this call.
 *
 *   q, out          : [B, Sq, Hq, D] (dtype);   lse : [B, Hq, Sq] fp32 (natural log,
 *                     +inf for a row that keeps no key)
 *   contiguous cache (block_table == NULL):
 *     k_cache, v_cache : [cache_batch, cache_seqlen, Hkv, D]; sequence b reads entry
 *                     cache_batch_idx[b] (int32 device array of B entries; NULL: entry b)
 *   paged cache (block_table != NULL):
 *     k_cache, v_cache : [num_blocks = cache_batch, page_block_size = cache_seqlen, Hkv, D];
 *     block_table : int32 device array [B, max_blocks_per_seq]; key j of sequence b is
 *     row j % page_block_size of block block_table[b * max_blocks_per_seq + j / page_block_size].
 *     page_block_size must be a multiple of 32.  cache_batch_idx must be NULL.
 *   cache_seqlens  : int32 device array of B lengths, or NULL for "every addressable key"
 *                    (cache_seqlen, or max_blocks_per_seq * page_block_size).  Lengths are
 *                    clamped to [0, that capacity] on the device.
 *   causal / window_left / window_right : bottom-right aligned with seqlen_k =
 *                    cache_seqlens[b]: query i keeps key j iff
 *                    i + Lk - Sq - window_left <= j <= i + Lk - Sq + window_right
 *                    (-1 = unbounded side) and, if causal, j <= i + Lk - Sq.
 *   alibi_slopes   : NULL, or fp32 device array; the slope of (b, h) is
 *                    alibi_slopes[b * alibi_batch_stride + h] (stride 0: one slope per
 *                    head; stride Hq: per sequence and head).  Adds
 *                    -slope * |i + Lk - Sq - j| to the scaled score.
 *   num_splits     : number of key ranges per (sequence, KV head); 0 picks a count
 *                    from the same rule as fa_fwd_kvcache_num_splits(...) applied to the
 *                    keys the window can reach, never more than that function returns
 *                    (so a workspace sized with it suffices).  With more than one split the
 *                    partial results go through `workspace`, which must hold
 *                    fa_fwd_kvcache_workspace_bytes(B, Sq, Hq, D, splits) bytes (16-byte
 *                    aligned; contents on entry do not matter); one split writes out and
 *                    lse directly and needs no workspace.
 * Device-side values (lengths, indices, block-table entries) are preconditions: indices
 * must address existing cache entries and blocks.  Errors as for fa_fwd.
 */
int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                   int B, int Sq, int Hq, int Hkv, int D, int cache_batch, int cache_seqlen,
                   const int32_t* cache_seqlens, const int32_t* cache_batch_idx,
                   const int32_t* block_table, int max_blocks_per_seq,
                   float scale, int causal, int window_left, int window_right,
                   const float* alibi_slopes, int alibi_batch_stride,
                   int num_splits, int dtype, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * Split count fa_fwd_kvcache uses for num_splits = 0: enough (sequence, KV head, split)
 * work items to fill the GPU, at least 256 keys per split, and (paged caches) few enough
 * pages per split.  seqlen_k is the cache capacity per sequence; page_block_size is 0 for
 * a contiguous cache.  Returns 1 for invalid sizes.
 */
int fa_fwd_kvcache_num_splits(int B, int Sq, int Hq, int Hkv, int D, int seqlen_k, int page_block_size);

/* Workspace bytes fa_fwd_kvcache needs for num_splits splits (0 when num_splits <= 1). */
size_t fa_fwd_kvcache_workspace_bytes(int B, int Sq, int Hq, int D, int num_splits);

/* Size of the static scratch array of fa_fwd_kvcache_noalloc, per device. */
#define FA_KVCACHE_NOALLOC_MAX_BYTES (64u << 20)

/*
 * fa_fwd_kvcache without a workspace, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The split partials go to a static device array of the library,
 * FA_KVCACHE_NOALLOC_MAX_BYTES bytes on each device it runs on, held until the process
 * ends; this call allocates nothing.  num_splits = 0 picks the fa_fwd_kvcache count,
 * lowered until the partials fit the array (one split needs none); an explicit count
 * whose partials (fa_fwd_kvcache_workspace_bytes) exceed it returns FA_ERR_WORKSPACE, as
 * does a paged cache whose smallest allowed count does not fit.  Every partial is written
 * by the split kernel before the merge reads it, so the array's contents on entry do not
 * matter.  All calls on one device share its array: calls that overlap in time on one
 * GPU (streams without an ordering between them) race and must not be issued.  Other
 * arguments, results and errors as for fa_fwd_kvcache.
 */
int fa_fwd_kvcache_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                           int B, int Sq, int Hq, int Hkv, int D, int cache_batch, int cache_seqlen,
                           const int32_t* cache_seqlens, const int32_t* cache_batch_idx,
                           const int32_t* block_table, int max_blocks_per_seq,
                           float scale, int causal, int window_left, int window_right,
                           const float* alibi_slopes, int alibi_batch_stride,
                           int num_splits, int dtype, hipStream_t stream);

/*
 * Result of the device-side argument checks (FA_DEBUG_CHECKS=1) on the current device:
 * synchronises `stream`, then returns FA_OK if no check has failed since the last report,
 * else FA_ERR_INVALID_ARGUMENT with fa_last_error() naming the failed checks, and clears
 * the flag.  While the flag is set every kernel of the library on that device returns at
 * once without writing its outputs.  Without FA_DEBUG_CHECKS=1 no check runs and this
 * returns FA_OK.  Unlike the other calls this one synchronises the host, so it cannot be
 * captured into a HIP graph.
 */
int fa_debug_status(hipStream_t stream);

/* Static description of a status code. */
const char* fa_status_string(int status);

/* Message describing the last error on the calling thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
