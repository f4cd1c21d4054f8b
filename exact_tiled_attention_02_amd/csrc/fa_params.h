// Kernel argument blocks and launcher declarations shared by the host library and the
// kernel translation units.  All sizes are validated by the host before a launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

// Codes of the device-side argument checks (FA_DEBUG_CHECKS=1), OR-ed into the flag.
constexpr int kDbgSeqlensStart = 1;   // cu_seqlens_q[0] or cu_seqlens_k[0] is not 0
constexpr int kDbgSeqlensOrder = 2;   // cu_seqlens decreases somewhere
constexpr int kDbgSeqlensQ = 4;       // a query sequence is longer than max_seqlen_q (Sq)
constexpr int kDbgSeqlensK = 8;       // a key sequence is longer than max_seqlen_k (Sk)
constexpr int kDbgCacheSeqlens = 16;  // cache_seqlens outside [0, capacity]
constexpr int kDbgCacheIndex = 32;    // cache_batch_idx outside [0, cache_batch)
constexpr int kDbgBlockTable = 64;    // a block-table entry outside [0, num_blocks)

struct FwdArgs {
  const int* dbg;  // device flag of the argument checks (null: checks off); set = do nothing
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
  const int* dbg;  // as in FwdArgs
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
  // Stored dS / scale in the input dtype (the route without dQ atomics), or null: one tile
  // of 32 query rows x KB keys (KB = keys per main-loop workgroup: 256 up to a 128-wide
  // tile, 128 above) per (sequence, query head, query step, key block), tile index
  // ((b * Hq + h) * ds_nqs + step) * ds_nkb + key block.  Inside a tile, the 32 keys of
  // main-loop wavefront w take bytes [2048 w, 2048 w + 2048): key row j (64 bytes) holds
  // the 32 rows at positions p, row = 16 ((p >> 3) & 1) + 8 ((p >> 2) & 1) + 4 (p >> 4) + (p & 3)
  // (the order in which the products leave them in a lane).
  uint16_t* ds;
  int ds_nqs;  // ceil(Sq / 32)
  int ds_nkb;  // ceil(Sk / KB)
};

// Decode against a read-only KV cache (few query rows, long cache), split over the keys.
struct DecodeArgs {
  const int* dbg;       // as in FwdArgs
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

// Device address of this device's argument-check flag (created on first use).
hipError_t debug_flag(int** out);
// One-workgroup check kernels (FA_DEBUG_CHECKS=1): OR a kDbg* code into *flag.
hipError_t launch_check_varlen(const int32_t* cu_q, const int32_t* cu_k, int B, int Sq, int Sk, int* flag,
                               hipStream_t stream);
hipError_t launch_check_kvcache(const int32_t* cache_seqlens, const int32_t* batch_idx, const int32_t* block_table,
                                int B, int cache_batch, int cap, int page, int max_blocks, int* flag,
                                hipStream_t stream);

// Device address of this device's static scratch array of fa_fwd_kvcache_noalloc
// (FA_KVCACHE_NOALLOC_MAX_BYTES, looked up once per device on first use).
hipError_t kvcache_scratch(void** out);

// Tile width of the kernels that serve head dimension D (D % 8 == 0, 8 <= D <= 256): the
// next of 64, 128, 256; 0 for anything else.
constexpr int tile_headdim(int D) {
  return (D <= 0 || D > 256 || D % 8 != 0) ? 0 : D <= 64 ? 64 : D <= 128 ? 128 : 256;
}

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// stage_mask bit 0: preprocess, bit 1: main loop with dQ atomics, bit 2: finalize,
// bit 3: deterministic dQ (main loop without dQ, then a separate dQ pass writing dq),
// bit 4: main loop without dQ that stores dS (a.ds), bit 5: dQ = scale dS K from the
// stored dS, written to dq.
constexpr int kBwdPre = 1, kBwdMainAtomic = 2, kBwdFinalize = 4, kBwdRecompute = 8, kBwdMainStoreDs = 16,
              kBwdDqFromDs = 32;
// Keys per backward main-loop workgroup for tile width D (the key-block size of the
// stored dS tiles).
constexpr int bwd_block_keys(int D) { return D <= 128 ? 256 : 128; }
hipError_t launch_bwd(const BwdArgs& a, int stage_mask, hipStream_t stream);
// Split kernel, then (splits > 1) the combine kernel.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// LDS ring depth (32-key stages) of the decode kernel for head dimension D: 48 KiB for
// D = 64 and 128 (three single-wavefront workgroups per CU), 64 KiB for D = 256.
constexpr int decode_stages(int D) { return D == 64 ? 6 : D == 128 ? 3 : 2; }

}  // namespace fa
