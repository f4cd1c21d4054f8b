// Device-side argument checks, enabled with FA_DEBUG_CHECKS=1 in the environment.
//
// Some preconditions live in device memory, where the host cannot read them without a
// synchronisation: the cu_seqlens offsets of a packed (varlen) batch (the
// kernels-community/flash-attn2 repository card, "Low-level ops", and the
// flash_attn_varlen_func arguments: cu_seqlens starts at 0 and is non-decreasing, every
// sequence is at most max_seqlen long) and the cache indices and block-table entries of a
// KV-cache call (flash_attn_with_kvcache docstring).  With the checks on, a one-workgroup
// kernel validates them on the call's stream before the attention kernels and ORs a
// code into a per-device flag; every attention kernel reads the flag first and does
// nothing when it is set.  fa_debug_status() reports (and clears) the flag after a
// synchronisation.  The flag is sticky: once set, later calls on the device skip their
// work too until it is reported.
#include <mutex>

#include "fa.h"
#include "fa_device.h"
#include "fa_params.h"

namespace fa {
namespace {

// One flag per device: each GPU the library runs on holds its own copy of this variable.
__device__ __align__(16) int g_debug_flag;

__global__ __launch_bounds__(256) void check_varlen_kernel(const int32_t* cu_q, const int32_t* cu_k, int B, int Sq,
                                                           int Sk, int* flag) {
  int bits = 0;
  if (threadIdx.x == 0 && (cu_q[0] != 0 || cu_k[0] != 0)) bits |= kDbgSeqlensStart;
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int lq = cu_q[b + 1] - cu_q[b];
    const int lk = cu_k[b + 1] - cu_k[b];
    if (lq < 0 || lk < 0) bits |= kDbgSeqlensOrder;
    if (lq > Sq) bits |= kDbgSeqlensQ;
    if (lk > Sk) bits |= kDbgSeqlensK;
  }
  if (bits) atomicOr(flag, bits);
}

__global__ __launch_bounds__(256) void check_kvcache_kernel(const int32_t* cache_seqlens, const int32_t* batch_idx,
                                                            const int32_t* block_table, int B, int cache_batch,
                                                            int cap, int page, int max_blocks, int* flag) {
  int bits = 0;
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    int Lk = cap;
    if (cache_seqlens != nullptr) {
      Lk = cache_seqlens[b];
      if (Lk < 0 || Lk > cap) bits |= kDbgCacheSeqlens;
      Lk = min(max(Lk, 0), cap);
    }
    if (batch_idx != nullptr && (batch_idx[b] < 0 || batch_idx[b] >= cache_batch)) bits |= kDbgCacheIndex;
    if (block_table != nullptr) {
      const int pages = (Lk + page - 1) / page;
      for (int p = 0; p < pages && p < max_blocks; ++p) {
        const int e = block_table[(size_t)b * max_blocks + p];
        if (e < 0 || e >= cache_batch) bits |= kDbgBlockTable;
      }
    }
  }
  if (bits) atomicOr(flag, bits);
}

std::mutex g_flag_mu;
int* g_flag_ptr[64];

}  // namespace

hipError_t debug_flag(int** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_flag_mu);
  if (g_flag_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_debug_flag));
    if (e != hipSuccess) return e;
    g_flag_ptr[dev] = static_cast<int*>(p);
  }
  *out = g_flag_ptr[dev];
  return hipSuccess;
}

hipError_t launch_check_varlen(const int32_t* cu_q, const int32_t* cu_k, int B, int Sq, int Sk, int* flag,
                               hipStream_t stream) {
  hipLaunchKernelGGL(check_varlen_kernel, dim3(1), dim3(256), 0, stream, cu_q, cu_k, B, Sq, Sk, flag);
  return hipGetLastError();
}

hipError_t launch_check_kvcache(const int32_t* cache_seqlens, const int32_t* batch_idx, const int32_t* block_table,
                                int B, int cache_batch, int cap, int page, int max_blocks, int* flag,
                                hipStream_t stream) {
  hipLaunchKernelGGL(check_kvcache_kernel, dim3(1), dim3(256), 0, stream, cache_seqlens, batch_idx, block_table, B,
                     cache_batch, cap, page, max_blocks, flag);
  return hipGetLastError();
}

}  // namespace fa
