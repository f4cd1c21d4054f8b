// Host side of libfa.so: argument validation, kernel choice and launch (C ABI of fa.h).
// Nothing here synchronises the host or allocates device memory.
#include "fa.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "fa_params.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by the forward and the backward.  Returns FA_OK or an error status.
int check_common(int B, int Sq, int Sk, int Hq, int Hkv, int D, float scale, const int32_t* cu_q,
                 const int32_t* cu_k, int dtype) {
  if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_UNSUPPORTED, "dtype %d is neither FA_DTYPE_FP16 nor FA_DTYPE_BF16", dtype);
  if (B <= 0 || Sq <= 0 || Sk <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "sizes must be positive (B=%d Sq=%d Sk=%d Hq=%d Hkv=%d D=%d)", B, Sq, Sk, Hq,
                Hkv, D);
  if (Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "Hq=%d is not divisible by Hkv=%d", Hq, Hkv);
  if (fa::tile_headdim(D) == 0)
    return fail(FA_ERR_UNSUPPORTED, "head dimension %d is not a multiple of 8 in [8, 256]", D);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(FA_ERR_INVALID_ARGUMENT, "scale must be finite and non-negative (got %g)", (double)scale);
  if ((cu_q == nullptr) != (cu_k == nullptr))
    return fail(FA_ERR_INVALID_ARGUMENT, "give both cu_seqlens_q and cu_seqlens_k, or neither");
  if (cu_q != nullptr && ((reinterpret_cast<uintptr_t>(cu_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_k) & 3u)))
    return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
  // Element counts must fit the 64-bit index math and the grid: rows * heads * D.
  const double rows_q = (double)B * Sq, rows_k = (double)B * Sk;
  if (rows_q * Hq * D > 9.0e15 || rows_k * Hkv * D > 9.0e15 || rows_q > 2147483647.0 || rows_k > 2147483647.0)
    return fail(FA_ERR_INVALID_ARGUMENT, "problem too large");
  return FA_OK;
}

// Window and ALiBi arguments shared by every entry point that takes them.
int check_mask_args(int window_left, int window_right, const float* alibi_slopes, int alibi_batch_stride, int Hq) {
  if (window_left < -1 || window_right < -1)
    return fail(FA_ERR_INVALID_ARGUMENT, "window sizes must be >= -1 (got %d, %d)", window_left, window_right);
  if (alibi_slopes && (reinterpret_cast<uintptr_t>(alibi_slopes) & 3u))
    return fail(FA_ERR_INVALID_ARGUMENT, "alibi_slopes must be 4-byte aligned");
  if (alibi_slopes && alibi_batch_stride != 0 && alibi_batch_stride != Hq)
    return fail(FA_ERR_INVALID_ARGUMENT, "alibi_batch_stride must be 0 or Hq (got %d)", alibi_batch_stride);
  return FA_OK;
}

// A window side at least as long as the sequences can reach is no limit at all: query i
// of a sequence with Lq <= Sq queries and Lk <= Sk keys keeps j >= i + Lk - Lq - left,
// which holds for every j >= 0 once left >= Sk, and j <= i + Lk - Lq + right, which holds
// for every j < Lk once right >= Sq.  Mapping those to -1 keeps the kernels' index
// arithmetic far from overflow.
int norm_left(int wl, int Sk) { return wl >= Sk ? -1 : wl; }
int norm_right(int wr, int Sq) { return wr >= Sq ? -1 : wr; }

int check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(FA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return FA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FA_OK;
  return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr float kLog2e = 1.4426950408889634f;

// FA_DEBUG_CHECKS=1 in the environment turns on the device-side argument checks.
bool debug_checks_on() {
  const char* e = std::getenv("FA_DEBUG_CHECKS");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

// With the checks on: the device flag every kernel of the call reads, after launching the
// check of the varlen offsets (when given).  Returns FA_OK (flag null when checks are off)
// or an error status.
int debug_setup(const int32_t* cu_q, const int32_t* cu_k, int B, int Sq, int Sk, hipStream_t stream,
                const int** flag_out) {
  *flag_out = nullptr;
  if (!debug_checks_on()) return FA_OK;
  int* flag = nullptr;
  int st = hip_status(fa::debug_flag(&flag), "FA_DEBUG_CHECKS flag");
  if (st != FA_OK) return st;
  if (cu_q != nullptr) {
    st = hip_status(fa::launch_check_varlen(cu_q, cu_k, B, Sq, Sk, flag, stream), "FA_DEBUG_CHECKS launch");
    if (st != FA_OK) return st;
  }
  *flag_out = flag;
  return FA_OK;
}

// Factor applied to raw scores before exp2: scale * log2(e), but at least 1e-30 so that
// it is strictly positive.  The kernels then mask a score by setting it to -inf
// (exp2(-inf * c) = 0 needs c > 0).  For scale = 0 the clamp changes nothing: every
// |score * 1e-30| is far below half an ulp of 1, so each kept weight is exactly 1.0f, as
// with a zero scale; the LSE and the gradients use the true scale.
float exp2_scale(float scale) {
  const float c = scale * kLog2e;
  return c < 1e-30f ? 1e-30f : c;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "unknown fa_status";
  }
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

int fa_debug_status(hipStream_t stream) {
  g_last_error.clear();
  int* flag = nullptr;
  int st = hip_status(fa::debug_flag(&flag), "FA_DEBUG_CHECKS flag");
  if (st != FA_OK) return st;
  int code = 0;
  if ((st = hip_status(hipMemcpyAsync(&code, flag, sizeof code, hipMemcpyDeviceToHost, stream), "read flag")) ||
      (st = hip_status(hipStreamSynchronize(stream), "synchronise")))
    return st;
  if (code == 0) return FA_OK;
  const int zero = 0;
  if ((st = hip_status(hipMemcpyAsync(flag, &zero, sizeof zero, hipMemcpyHostToDevice, stream), "clear flag")) ||
      (st = hip_status(hipStreamSynchronize(stream), "synchronise")))
    return st;
  std::string msg = "device-side argument check failed (code " + std::to_string(code) + "):";
  if (code & fa::kDbgSeqlensStart) msg += " cu_seqlens does not start at 0;";
  if (code & fa::kDbgSeqlensOrder) msg += " cu_seqlens decreases;";
  if (code & fa::kDbgSeqlensQ) msg += " a query sequence is longer than max_seqlen_q;";
  if (code & fa::kDbgSeqlensK) msg += " a key sequence is longer than max_seqlen_k;";
  if (code & fa::kDbgCacheSeqlens) msg += " cache_seqlens outside [0, capacity];";
  if (code & fa::kDbgCacheIndex) msg += " cache_batch_idx outside the cache;";
  if (code & fa::kDbgBlockTable) msg += " a block-table entry outside the block pool;";
  g_last_error = msg;
  return FA_ERR_INVALID_ARGUMENT;
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Sq, int Sk, int Hq,
              int Hkv, int D, float scale, int causal, int window_left, int window_right, const float* alibi_slopes,
              int alibi_batch_stride, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype,
              hipStream_t stream) {
  g_last_error.clear();
  int st = check_common(B, Sq, Sk, Hq, Hkv, D, scale, cu_seqlens_q, cu_seqlens_k, dtype);
  if (st != FA_OK) return st;
  if ((st = check_mask_args(window_left, window_right, alibi_slopes, alibi_batch_stride, Hq))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(out, "out")) || (st = check_ptr(lse, "lse")))
    return st;
  fa::FwdArgs a{};
  if ((st = debug_setup(cu_seqlens_q, cu_seqlens_k, B, Sq, Sk, stream, &a.dbg))) return st;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.B = B;
  a.Sq = Sq;
  a.Sk = Sk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.causal = causal ? 1 : 0;
  a.window_left = norm_left(window_left, Sk);
  a.window_right = norm_right(window_right, Sq);
  a.alibi = alibi_slopes;
  a.alibi_bstride = alibi_batch_stride;
  a.bf16 = dtype == FA_DTYPE_BF16;
  a.scale = scale;
  a.scale_log2 = exp2_scale(scale);
  return hip_status(fa::launch_fwd(a, stream), "fa_fwd launch");
}

int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Sq, int Sk, int Hq, int Hkv,
           int D, float scale, int causal, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype,
           hipStream_t stream) {
  return fa_fwd_ex(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, scale, causal, -1, -1, nullptr, 0, cu_seqlens_q,
                   cu_seqlens_k, dtype, stream);
}

size_t fa_bwd_workspace_bytes(int B, int Sq, int Hq, int D) {
  if (B <= 0 || Sq <= 0 || Hq <= 0 || D <= 0) return 0;
  const size_t rows = (size_t)B * Sq;
  const size_t acc = rows * Hq * D * sizeof(float);
  const size_t dsum = rows * Hq * sizeof(float);
  // Dsum and LSE*log2(e) (dsum bytes each), then 256 bytes: the two counters of the main
  // loop's key-block queue
  return ((acc + 255) & ~(size_t)255) + 2 * ((dsum + 255) & ~(size_t)255) + 256;
}

size_t fa_bwd_ds_workspace_bytes(int B, int Sq, int Sk, int Hq, int D) {
  const int tile = fa::tile_headdim(D);
  if (B <= 0 || Sq <= 0 || Sk <= 0 || Hq <= 0 || tile == 0) return 0;
  const int kb = fa::bwd_block_keys(tile);
  const size_t tiles = (size_t)B * Hq * (size_t)((Sq + 31) / 32) * (size_t)((Sk + kb - 1) / kb);
  const size_t bytes = tiles * 32 * kb * 2;
  return bytes > FA_BWD_DS_MAX_BYTES ? 0 : (bytes + 255) & ~(size_t)255;
}

namespace {

// Stages of a whole backward: preprocess, then, when the workspace holds the stored-dS
// area, the main loop that stores dS followed by dQ from it (no atomics, no second
// computation of S and dP: the fastest route, and deterministic); otherwise either the main
// loop with dQ atomics and the finalize, or the main loop without dQ followed by the dQ
// pass that recomputes S and dP.  Above a 128-wide tile the atomic route is the slower of
// those two (its main loop covers 128 keys per workgroup, so it issues one fp32 atomic per
// dQ element per 128 keys, and the memory-side atomic rate bounds it: B=1 H=16 S=8192
// D=256 causal 5.3 ms against 3.1 ms for the two passes), so there the recompute route
// serves the default backward too.
// At tile width 64 the stored-dS route moves the same 4 bytes of dS per (row, key) pair as at
// 128 for half the products, and the atomic route issues half the atomics per pair: there
// the atomic route is the faster one (hidden 2048 as 32 heads of 64, S = 16k: 7.2 ms
// against 10.3 ms), so fa_bwd keeps it even when the workspace holds the dS area; the
// deterministic call still takes the stored-dS route, which avoids the second computation
// of S and dP.
int full_bwd_stages(int D, bool deterministic, bool stored_ds) {
  if (stored_ds && (deterministic || fa::tile_headdim(D) >= 128))
    return fa::kBwdPre | fa::kBwdMainStoreDs | fa::kBwdDqFromDs;
  return deterministic || fa::tile_headdim(D) > 128 ? (fa::kBwdPre | fa::kBwdRecompute)
                                                    : (fa::kBwdPre | fa::kBwdMainAtomic | fa::kBwdFinalize);
}

// Whether a backward with this workspace takes the stored-dS route.
bool has_ds_area(int B, int Sq, int Sk, int Hq, int D, size_t workspace_bytes) {
  const size_t ds = fa_bwd_ds_workspace_bytes(B, Sq, Sk, Hq, D);
  const size_t base = fa_bwd_workspace_bytes(B, Sq, Hq, D);
  return ds > 0 && base > 0 && workspace_bytes >= ((base + 255) & ~(size_t)255) + ds;
}

int bwd_impl(int stage_mask, const void* dout, const void* q, const void* k, const void* v, const void* out,
             const float* lse, void* dq, void* dk, void* dv, int B, int Sq, int Sk, int Hq, int Hkv, int D,
             float scale, int causal, int window_left, int window_right, const float* alibi_slopes,
             int alibi_batch_stride, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype,
             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  int st = check_common(B, Sq, Sk, Hq, Hkv, D, scale, cu_seqlens_q, cu_seqlens_k, dtype);
  if (st != FA_OK) return st;
  if ((st = check_mask_args(window_left, window_right, alibi_slopes, alibi_batch_stride, Hq))) return st;
  if ((st = check_ptr(dout, "dout")) || (st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) ||
      (st = check_ptr(v, "v")) || (st = check_ptr(out, "out")) || (st = check_ptr(lse, "lse")) ||
      (st = check_ptr(dq, "dq")) || (st = check_ptr(dk, "dk")) || (st = check_ptr(dv, "dv")))
    return st;
  // The backward main loop addresses a block of 256 keys with 31-bit lane offsets.
  if ((long long)Hkv * D * 2 * 256 >= (1LL << 31))
    return fail(FA_ERR_UNSUPPORTED, "Hkv * D = %lld is too wide for the backward (limit 2^22)", (long long)Hkv * D);
  const size_t need = fa_bwd_workspace_bytes(B, Sq, Hq, D);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu at %p)", need,
                workspace_bytes, workspace);
  fa::BwdArgs a{};
  if ((st = debug_setup(cu_seqlens_q, cu_seqlens_k, B, Sq, Sk, stream, &a.dbg))) return st;
  a.dout = dout;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const size_t rows = (size_t)B * Sq;
  const size_t acc_bytes = (rows * Hq * D * sizeof(float) + 255) & ~(size_t)255;
  a.dq_acc = static_cast<float*>(workspace);
  a.dsum = reinterpret_cast<float*>(static_cast<char*>(workspace) + acc_bytes);
  const size_t dsum_bytes = (rows * Hq * sizeof(float) + 255) & ~(size_t)255;
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + acc_bytes + dsum_bytes);
  a.work = reinterpret_cast<unsigned int*>(static_cast<char*>(workspace) + acc_bytes + 2 * dsum_bytes);
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.B = B;
  a.Sq = Sq;
  a.Sk = Sk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.causal = causal ? 1 : 0;
  a.window_left = norm_left(window_left, Sk);
  a.window_right = norm_right(window_right, Sq);
  a.alibi = alibi_slopes;
  a.alibi_bstride = alibi_batch_stride;
  a.bf16 = dtype == FA_DTYPE_BF16;
  a.scale = scale;
  a.scale_log2 = exp2_scale(scale);
  // only the atomic dQ path uses the accumulator
  a.zero_acc = (stage_mask & (fa::kBwdRecompute | fa::kBwdMainStoreDs | fa::kBwdDqFromDs)) == 0;
  if (stage_mask & (fa::kBwdMainStoreDs | fa::kBwdDqFromDs)) {
    if (!has_ds_area(B, Sq, Sk, Hq, D, workspace_bytes))
      return fail(FA_ERR_WORKSPACE, "the stored-dS stages need %zu + %zu bytes of workspace (got %zu)",
                  (need + 255) & ~(size_t)255, fa_bwd_ds_workspace_bytes(B, Sq, Sk, Hq, D), workspace_bytes);
    const int kb = fa::bwd_block_keys(fa::tile_headdim(D));
    a.ds = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + ((need + 255) & ~(size_t)255));
    a.ds_nqs = (Sq + 31) / 32;
    a.ds_nkb = (Sk + kb - 1) / kb;
  }
  return hip_status(fa::launch_bwd(a, stage_mask, stream), "fa_bwd launch");
}

}  // namespace

int fa_bwd(const void* dout, const void* q, const void* k, const void* v, const void* out, const float* lse, void* dq,
           void* dk, void* dv, int B, int Sq, int Sk, int Hq, int Hkv, int D, float scale, int causal,
           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype, void* workspace,
           size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(full_bwd_stages(D, false, has_ds_area(B, Sq, Sk, Hq, D, workspace_bytes)), dout, q, k, v, out,
                  lse, dq, dk, dv, B, Sq, Sk, Hq, Hkv, D, scale, causal, -1, -1, nullptr, 0, cu_seqlens_q,
                  cu_seqlens_k, dtype, workspace, workspace_bytes, stream);
}

int fa_bwd_deterministic(const void* dout, const void* q, const void* k, const void* v, const void* out,
                         const float* lse, void* dq, void* dk, void* dv, int B, int Sq, int Sk, int Hq, int Hkv,
                         int D, float scale, int causal, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(full_bwd_stages(D, true, has_ds_area(B, Sq, Sk, Hq, D, workspace_bytes)), dout, q, k, v, out,
                  lse, dq, dk, dv, B, Sq, Sk, Hq, Hkv, D, scale, causal, -1, -1, nullptr, 0, cu_seqlens_q,
                  cu_seqlens_k, dtype, workspace, workspace_bytes, stream);
}

int fa_bwd_stage(int stage, const void* dout, const void* q, const void* k, const void* v, const void* out,
                 const float* lse, void* dq, void* dk, void* dv, int B, int Sq, int Sk, int Hq, int Hkv, int D,
                 float scale, int causal, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (stage < 1 || stage > 5) {
    g_last_error.clear();
    return fail(FA_ERR_INVALID_ARGUMENT, "stage %d is not 1, 2, 3, 4 or 5", stage);
  }
  static const int masks[5] = {fa::kBwdPre, fa::kBwdMainAtomic, fa::kBwdFinalize, fa::kBwdMainStoreDs,
                               fa::kBwdDqFromDs};
  return bwd_impl(masks[stage - 1], dout, q, k, v, out, lse, dq, dk, dv, B, Sq, Sk, Hq, Hkv, D, scale, causal, -1,
                  -1, nullptr, 0, cu_seqlens_q, cu_seqlens_k, dtype, workspace, workspace_bytes, stream);
}

int fa_bwd_ex(const void* dout, const void* q, const void* k, const void* v, const void* out, const float* lse,
              void* dq, void* dk, void* dv, int B, int Sq, int Sk, int Hq, int Hkv, int D, float scale, int causal,
              int window_left, int window_right, const float* alibi_slopes, int alibi_batch_stride,
              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype, int deterministic,
              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(full_bwd_stages(D, deterministic != 0, has_ds_area(B, Sq, Sk, Hq, D, workspace_bytes)), dout, q, k, v, out, lse, dq, dk, dv, B, Sq, Sk, Hq, Hkv, D, scale,
                  causal, window_left, window_right, alibi_slopes, alibi_batch_stride, cu_seqlens_q, cu_seqlens_k,
                  dtype, workspace, workspace_bytes, stream);
}

namespace {

int decode_row_groups(int Sq, int Hq, int Hkv) { return (int)(((long long)Sq * (Hq / Hkv) + 31) / 32); }

// Upper bound on the 32-key tiles one row group of a sequence can touch: the capacity, or
// with a left window the window's span over the Sq queries (plus one tile on each side
// for alignment).
int decode_span_tiles(int cap, int Sq, int causal, int wl, int wr) {
  const long long cap_tiles = (cap + 31) / 32;
  if (wl < 0) return (int)cap_tiles;
  const long long right = causal ? 0 : (wr >= 0 ? wr : (long long)cap);
  const long long keys = (long long)Sq + wl + right;
  return (int)std::min(cap_tiles, (keys + 31) / 32 + 1);
}

// Tiles per split for a given split count.
int decode_chunk(int span_tiles, int splits) { return (span_tiles + splits - 1) / splits; }

// Smallest split count for which no split of a paged cache touches more than 64 pages
// (the kernel keeps a split's page list in one register per lane).
int decode_min_splits(int span_tiles, int page) {
  if (page <= 0) return 1;
  for (int s = 1;; ++s) {
    const long long chunk = decode_chunk(span_tiles, s);
    if ((chunk * 32 + page - 1) / page + 1 <= 64) return s;
  }
}

int decode_splits_heuristic(long long units, int span_tiles, int page) {
  // About 4096 single-wavefront workgroups when every cache is full (five rounds of three
  // per CU on 256 CUs; shorter caches leave some splits empty, and small equal chunks
  // keep the rest balanced), at least 8 tiles (256 keys) per split, at most 1024 splits.
  long long s = (4096 + units - 1) / units;
  s = std::min<long long>(s, std::max(1, span_tiles / 8));
  s = std::min<long long>(s, 1024);
  s = std::max<long long>(s, decode_min_splits(span_tiles, page));
  return (int)std::max<long long>(s, 1);
}

}  // namespace

int fa_fwd_kvcache_num_splits(int B, int Sq, int Hq, int Hkv, int D, int seqlen_k, int page_block_size) {
  if (B <= 0 || Sq <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || seqlen_k <= 0) return 1;
  (void)D;
  const long long units = (long long)B * Hkv * decode_row_groups(Sq, Hq, Hkv);
  return decode_splits_heuristic(units, decode_span_tiles(seqlen_k, Sq, 0, -1, -1), page_block_size);
}

size_t fa_fwd_kvcache_workspace_bytes(int B, int Sq, int Hq, int D, int num_splits) {
  if (B <= 0 || Sq <= 0 || Hq <= 0 || D <= 0 || num_splits <= 1) return 0;
  const size_t rows = (size_t)num_splits * B * Sq * Hq;
  return ((rows * D * sizeof(float) + 255) & ~(size_t)255) + ((rows * sizeof(float) + 255) & ~(size_t)255);
}

}  // extern "C"

namespace {

// fa_fwd_kvcache; with noalloc the split partials go to the library's static scratch
// array instead of `workspace` (fa_fwd_kvcache_noalloc).
int kvcache_impl(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse, int B, int Sq,
                 int Hq, int Hkv, int D, int cache_batch, int cache_seqlen, const int32_t* cache_seqlens,
                 const int32_t* cache_batch_idx, const int32_t* block_table, int max_blocks_per_seq, float scale,
                 int causal, int window_left, int window_right, const float* alibi_slopes, int alibi_batch_stride,
                 int num_splits, int dtype, void* workspace, size_t workspace_bytes, bool noalloc,
                 hipStream_t stream) {
  g_last_error.clear();
  const bool paged = block_table != nullptr;
  const long long cap_ll = paged ? (long long)max_blocks_per_seq * cache_seqlen : (long long)cache_seqlen;
  int st = check_common(B, Sq, cap_ll > 0 && cap_ll < (1 << 30) ? (int)cap_ll : 1, Hq, Hkv, D, scale, nullptr,
                        nullptr, dtype);
  if (st != FA_OK) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k_cache, "k_cache")) || (st = check_ptr(v_cache, "v_cache")) ||
      (st = check_ptr(out, "out")) || (st = check_ptr(lse, "lse")))
    return st;
  if (cache_batch <= 0 || cache_seqlen <= 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "cache dimensions must be positive (%d, %d)", cache_batch, cache_seqlen);
  if (paged) {
    if (cache_batch_idx != nullptr)
      return fail(FA_ERR_INVALID_ARGUMENT, "cache_batch_idx cannot be combined with a block table");
    if (max_blocks_per_seq <= 0)
      return fail(FA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq must be positive (got %d)", max_blocks_per_seq);
    if (cache_seqlen % 32 != 0)
      return fail(FA_ERR_INVALID_ARGUMENT, "page_block_size must be a multiple of 32 (got %d)", cache_seqlen);
    if (reinterpret_cast<uintptr_t>(block_table) & 3u)
      return fail(FA_ERR_INVALID_ARGUMENT, "block_table must be 4-byte aligned");
  }
  if (cap_ll >= (1 << 30)) return fail(FA_ERR_INVALID_ARGUMENT, "KV cache longer than 2^30 keys per sequence");
  if ((double)cache_batch * cache_seqlen * Hkv * D > 9.0e15)
    return fail(FA_ERR_INVALID_ARGUMENT, "KV cache too large");
  if ((cache_seqlens && (reinterpret_cast<uintptr_t>(cache_seqlens) & 3u)) ||
      (cache_batch_idx && (reinterpret_cast<uintptr_t>(cache_batch_idx) & 3u)))
    return fail(FA_ERR_INVALID_ARGUMENT, "cache_seqlens and cache_batch_idx must be 4-byte aligned");
  if ((st = check_mask_args(window_left, window_right, alibi_slopes, alibi_batch_stride, Hq))) return st;
  const int cap = (int)cap_ll;
  window_left = norm_left(window_left, cap);
  window_right = norm_right(window_right, Sq);
  const int page = paged ? cache_seqlen : 0;
  if (num_splits < 0 || num_splits > 1024)
    return fail(FA_ERR_INVALID_ARGUMENT, "num_splits must be in [0, 1024] (got %d)", num_splits);
  const int span = decode_span_tiles(cap, Sq, causal, window_left, window_right);
  // With a window the span (and so the heuristic count) can only shrink, so a workspace
  // sized by fa_fwd_kvcache_num_splits is always large enough.
  const int min_splits = paged ? decode_min_splits(span, page) : 1;
  if (num_splits == 0) {
    num_splits = decode_splits_heuristic((long long)B * Hkv * decode_row_groups(Sq, Hq, Hkv), span, page);
    // Without a workspace: as many splits as the scratch array holds (one split needs none).
    if (noalloc)
      while (num_splits > min_splits &&
             fa_fwd_kvcache_workspace_bytes(B, Sq, Hq, D, num_splits) > FA_KVCACHE_NOALLOC_MAX_BYTES)
        --num_splits;
  }
  if (paged && num_splits < min_splits)
    return fail(FA_ERR_INVALID_ARGUMENT, "a paged cache of %d keys in pages of %d needs num_splits >= %d", cap, page,
                min_splits);
  const double items = (double)B * Hkv * num_splits * decode_row_groups(Sq, Hq, Hkv);
  if (items > 2.0e9) return fail(FA_ERR_INVALID_ARGUMENT, "too many work items");
  const size_t need = fa_fwd_kvcache_workspace_bytes(B, Sq, Hq, D, num_splits);
  if (noalloc && need > 0) {
    if (need > FA_KVCACHE_NOALLOC_MAX_BYTES)
      return fail(FA_ERR_WORKSPACE,
                  "%d splits need %zu bytes of partial results, more than the %u bytes of the static scratch array",
                  num_splits, need, (unsigned)FA_KVCACHE_NOALLOC_MAX_BYTES);
    if ((st = hip_status(fa::kvcache_scratch(&workspace), "kvcache scratch array"))) return st;
    workspace_bytes = FA_KVCACHE_NOALLOC_MAX_BYTES;
  }
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need))
    return fail(FA_ERR_WORKSPACE, "%d splits need %zu bytes of workspace, 16-byte aligned (got %zu at %p)",
                num_splits, need, workspace_bytes, workspace);
  fa::DecodeArgs a{};
  if ((st = debug_setup(nullptr, nullptr, B, Sq, cap, stream, &a.dbg))) return st;
  if (a.dbg != nullptr && (cache_seqlens || cache_batch_idx || block_table)) {
    st = hip_status(fa::launch_check_kvcache(cache_seqlens, cache_batch_idx, block_table, B, cache_batch, cap, page,
                                             paged ? max_blocks_per_seq : 0, const_cast<int*>(a.dbg), stream),
                    "FA_DEBUG_CHECKS launch");
    if (st != FA_OK) return st;
  }
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.lse = lse;
  if (need > 0) {
    const size_t rows = (size_t)num_splits * B * Sq * Hq;
    a.o_part = static_cast<float*>(workspace);
    a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          ((rows * D * sizeof(float) + 255) & ~(size_t)255));
  }
  a.cache_seqlens = cache_seqlens;
  a.cache_batch_idx = cache_batch_idx;
  a.block_table = block_table;
  a.alibi = alibi_slopes;
  a.alibi_bstride = alibi_batch_stride;
  a.B = B;
  a.Sq = Sq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.cap = cap;
  a.entry_stride = (long long)cache_seqlen * Hkv * D;
  a.page = page;
  a.max_blocks = paged ? max_blocks_per_seq : 0;
  a.causal = causal ? 1 : 0;
  a.window_left = window_left;
  a.window_right = window_right;
  a.bf16 = dtype == FA_DTYPE_BF16;
  a.scale = scale;
  a.scale_log2 = exp2_scale(scale);
  a.splits = num_splits;
  a.chunk_tiles = decode_chunk(span, num_splits);
  a.row_groups = decode_row_groups(Sq, Hq, Hkv);
  return hip_status(fa::launch_decode(a, stream), "fa_fwd_kvcache launch");
}

}  // namespace

extern "C" {

int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse, int B, int Sq,
                   int Hq, int Hkv, int D, int cache_batch, int cache_seqlen, const int32_t* cache_seqlens,
                   const int32_t* cache_batch_idx, const int32_t* block_table, int max_blocks_per_seq, float scale,
                   int causal, int window_left, int window_right, const float* alibi_slopes, int alibi_batch_stride,
                   int num_splits, int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return kvcache_impl(q, k_cache, v_cache, out, lse, B, Sq, Hq, Hkv, D, cache_batch, cache_seqlen, cache_seqlens,
                      cache_batch_idx, block_table, max_blocks_per_seq, scale, causal, window_left, window_right,
                      alibi_slopes, alibi_batch_stride, num_splits, dtype, workspace, workspace_bytes, false, stream);
}

int fa_fwd_kvcache_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse, int B,
                           int Sq, int Hq, int Hkv, int D, int cache_batch, int cache_seqlen,
                           const int32_t* cache_seqlens, const int32_t* cache_batch_idx, const int32_t* block_table,
                           int max_blocks_per_seq, float scale, int causal, int window_left, int window_right,
                           const float* alibi_slopes, int alibi_batch_stride, int num_splits, int dtype,
                           hipStream_t stream) {
  return kvcache_impl(q, k_cache, v_cache, out, lse, B, Sq, Hq, Hkv, D, cache_batch, cache_seqlen, cache_seqlens,
                      cache_batch_idx, block_table, max_blocks_per_seq, scale, causal, window_left, window_right,
                      alibi_slopes, alibi_batch_stride, num_splits, dtype, nullptr, 0, true, stream);
}

}  // extern "C"
