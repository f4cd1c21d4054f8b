// Kernel argument blocks and launcher declarations shared by the host library and the
// kernel translation units.  All sizes are validated by the host before a launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* cu_q;  // null in padded mode
  const int32_t* cu_k;
  int B, Sq, Sk, Hq, Hkv, D;
  int causal;
  int window_left;   // sliding window (-1: unbounded; normalised to < Sk, < Sq by the host)
  int window_right;
  const float* alibi;  // ALiBi slopes alibi[b * alibi_bstride + h], or null
  int alibi_bstride;
  int bf16;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
};

struct BwdArgs {
  const void* dout;
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dq_acc;  // fp32 [rows, Hq, D], rows = B*Sq (padded) or >= total_q (varlen)
  float* dsum;    // fp32 [rows, Hq]: -Dsum = -rowsum(dO * O) (preprocess)
  float* lse2;    // fp32 [rows, Hq]: LSE * log2(e), the exp2 offset of P (preprocess)
  const int32_t* cu_q;
  const int32_t* cu_k;
  int B, Sq, Sk, Hq, Hkv, D;
  int causal;
  int window_left;   // as in FwdArgs
  int window_right;
  const float* alibi;
  int alibi_bstride;
  int bf16;
  float scale;
  float scale_log2;
  int zero_acc;  // preprocess also zeroes dq_acc (the atomic path needs it)
  unsigned int* work;  // [2]: key blocks handed out, workgroups finished (zero between launches)
};

// Decode against a read-only KV cache (few query rows, long cache), split over the keys.
struct DecodeArgs {
  const void* q;        // [B, Sq, Hq, D]
  const void* k;        // cache: [cache_batch, cap, Hkv, D], or pages [num_blocks, page, Hkv, D]
  const void* v;
  void* out;            // [B, Sq, Hq, D]
  float* lse;           // [B, Hq, Sq]
  float* o_part;        // [splits, B*Sq*Hq, D] fp32 partial outputs (splits > 1)
  float* lse_part;      // [splits, B*Hq*Sq] fp32 partial LSE (natural log, -inf = no key)
  const int32_t* cache_seqlens;    // [B] or null (every sequence has cap keys)
  const int32_t* cache_batch_idx;  // [B] or null (sequence b reads cache entry b)
  const int32_t* block_table;      // [B, max_blocks] or null (contiguous cache)
  const float* alibi;              // slopes, alibi[b * alibi_bstride + h], or null
  int alibi_bstride;
  int B, Sq, Hq, Hkv, D;
  int cap;                // keys a sequence can address
  long long entry_stride; // elements between cache entries (contiguous cache)
  int page, max_blocks;   // paged cache
  int causal, window_left, window_right;
  int bf16;
  float scale, scale_log2;
  int splits;
  int chunk_tiles;        // 32-key tiles per split; splits * chunk_tiles covers every range
  int row_groups;         // ceil(Sq * Hq / Hkv / 32)
};

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// stage_mask bit 0: preprocess, bit 1: main loop with dQ atomics, bit 2: finalize,
// bit 3: deterministic dQ (main loop without dQ, then a separate dQ pass writing dq).
hipError_t launch_bwd(const BwdArgs& a, int stage_mask, hipStream_t stream);
// Split kernel, then (splits > 1) the combine kernel.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// LDS ring depth (32-key stages) of the decode kernel for head dimension D: 48 KiB for
// D = 64 and 128 (three single-wavefront workgroups per CU), 64 KiB for D = 256.
constexpr int decode_stages(int D) { return D == 64 ? 6 : D == 128 ? 3 : 2; }

}  // namespace fa
