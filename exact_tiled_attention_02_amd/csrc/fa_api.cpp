// Host side of libfa.so: argument validation, kernel choice and launch (C ABI of fa.h).
// Nothing here synchronises the host or allocates device memory.
#include "fa.h"

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
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
  if (D != 64 && D != 128 && D != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dimension %d has no kernel (64, 128, 256)", D);
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

int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Sq, int Sk, int Hq, int Hkv,
           int D, float scale, int causal, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype,
           hipStream_t stream) {
  g_last_error.clear();
  int st = check_common(B, Sq, Sk, Hq, Hkv, D, scale, cu_seqlens_q, cu_seqlens_k, dtype);
  if (st != FA_OK) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(out, "out")) || (st = check_ptr(lse, "lse")))
    return st;
  fa::FwdArgs a{};
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
  a.bf16 = dtype == FA_DTYPE_BF16;
  a.scale = scale;
  a.scale_log2 = exp2_scale(scale);
  return hip_status(fa::launch_fwd(a, stream), "fa_fwd launch");
}

size_t fa_bwd_workspace_bytes(int B, int Sq, int Hq, int D) {
  if (B <= 0 || Sq <= 0 || Hq <= 0 || D <= 0) return 0;
  const size_t rows = (size_t)B * Sq;
  const size_t acc = rows * Hq * D * sizeof(float);
  const size_t dsum = rows * Hq * sizeof(float);
  return ((acc + 255) & ~(size_t)255) + ((dsum + 255) & ~(size_t)255);
}

namespace {

int bwd_impl(int stage_mask, const void* dout, const void* q, const void* k, const void* v, const void* out,
             const float* lse, void* dq, void* dk, void* dv, int B, int Sq, int Sk, int Hq, int Hkv, int D,
             float scale, int causal, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype,
             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  int st = check_common(B, Sq, Sk, Hq, Hkv, D, scale, cu_seqlens_q, cu_seqlens_k, dtype);
  if (st != FA_OK) return st;
  if ((st = check_ptr(dout, "dout")) || (st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) ||
      (st = check_ptr(v, "v")) || (st = check_ptr(out, "out")) || (st = check_ptr(lse, "lse")) ||
      (st = check_ptr(dq, "dq")) || (st = check_ptr(dk, "dk")) || (st = check_ptr(dv, "dv")))
    return st;
  const size_t need = fa_bwd_workspace_bytes(B, Sq, Hq, D);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu at %p)", need,
                workspace_bytes, workspace);
  fa::BwdArgs a{};
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
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.B = B;
  a.Sq = Sq;
  a.Sk = Sk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.causal = causal ? 1 : 0;
  a.bf16 = dtype == FA_DTYPE_BF16;
  a.scale = scale;
  a.scale_log2 = exp2_scale(scale);
  a.zero_acc = (stage_mask & 8) == 0;  // only the atomic dQ path uses the accumulator
  return hip_status(fa::launch_bwd(a, stage_mask, stream), "fa_bwd launch");
}

}  // namespace

int fa_bwd(const void* dout, const void* q, const void* k, const void* v, const void* out, const float* lse, void* dq,
           void* dk, void* dv, int B, int Sq, int Sk, int Hq, int Hkv, int D, float scale, int causal,
           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype, void* workspace,
           size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(7, dout, q, k, v, out, lse, dq, dk, dv, B, Sq, Sk, Hq, Hkv, D, scale, causal, cu_seqlens_q,
                  cu_seqlens_k, dtype, workspace, workspace_bytes, stream);
}

int fa_bwd_deterministic(const void* dout, const void* q, const void* k, const void* v, const void* out,
                         const float* lse, void* dq, void* dk, void* dv, int B, int Sq, int Sk, int Hq, int Hkv,
                         int D, float scale, int causal, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(1 | 8, dout, q, k, v, out, lse, dq, dk, dv, B, Sq, Sk, Hq, Hkv, D, scale, causal, cu_seqlens_q,
                  cu_seqlens_k, dtype, workspace, workspace_bytes, stream);
}

int fa_bwd_stage(int stage, const void* dout, const void* q, const void* k, const void* v, const void* out,
                 const float* lse, void* dq, void* dk, void* dv, int B, int Sq, int Sk, int Hq, int Hkv, int D,
                 float scale, int causal, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (stage < 1 || stage > 3) {
    g_last_error.clear();
    return fail(FA_ERR_INVALID_ARGUMENT, "stage %d is not 1, 2 or 3", stage);
  }
  return bwd_impl(1 << (stage - 1), dout, q, k, v, out, lse, dq, dk, dv, B, Sq, Sk, Hq, Hkv, D, scale, causal,
                  cu_seqlens_q, cu_seqlens_k, dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"
