// Measurement program (not part of libfa.so): the LDS read rate of one CU on MI355X for the
// read forms the attention kernels use -- 16-byte rows (ds_read_b128, the MFMA operand
// reads of Q and K), the transposing ds_read_b64_tr_b16 (V and the backward's transposed
// tiles) and plain 8-byte reads.  One 512-thread workgroup per CU; every wavefront streams
// conflict-free reads from a 96 KB LDS array (all addresses inside it) and folds the data
// into two registers so that no read is dead.  Cycles come from s_memtime of wavefront 0.
// Prints one JSON line per read form.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

#include "fa_device.h"

namespace {

constexpr int kElems = 6144;  // 16-byte elements: 96 KB, so one workgroup per CU
constexpr int kIters = 4096;  // 16 reads per wavefront per iteration

template <int MODE>
__global__ __launch_bounds__(512) void lds_rate_kernel(unsigned long long* cycles, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint4 buf[kElems];
  for (int i = threadIdx.x; i < kElems; i += 512) buf[i] = make_uint4(i, i * 3u, i * 5u, i * 7u);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  uint32_t x0 = 0, x1 = 0;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kIters; ++it) {
    // the window moves every iteration, so no read repeats the one before it; its
    // furthest element, base + 16 * 64 + 63 16-byte elements, stays below kElems
    const int base = (it & 3) * 1024;
    if constexpr (MODE == 0) {  // ds_read_b128: 1 KB per wavefront instruction
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint4 v = buf[base + u * 64 + lane];
        x0 ^= v.x ^ v.y;
        x1 ^= v.z ^ v.w;
      }
    } else if constexpr (MODE == 1) {  // ds_read_b64_tr_b16: 512 B per instruction
      const uint16_t* p = reinterpret_cast<const uint16_t*>(buf + base);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const fa::u32x2 v = fa::lds_read_tr16(p + u * 256 + lane * 4);
        x0 ^= v.x;
        x1 ^= v.y;
      }
    } else {  // 8-byte reads: 512 B per instruction
      const uint2* p = reinterpret_cast<const uint2*>(buf + base);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint2 v = p[u * 64 + lane];
        x0 ^= v.x;
        x1 ^= v.y;
      }
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
  sink[blockIdx.x * 512 + threadIdx.x] = x0 ^ x1;
}

bool ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return false;
}

template <int MODE>
bool measure(int ncu, unsigned long long* cycles, uint32_t* sink, const char* name, int bytes_per_read) {
  for (int w = 0; w < 3; ++w) hipLaunchKernelGGL(lds_rate_kernel<MODE>, dim3(ncu), dim3(512), 0, 0, cycles, sink);
  hipEvent_t e0, e1;
  if (!ok(hipEventCreate(&e0), "event") || !ok(hipEventCreate(&e1), "event")) return false;
  if (!ok(hipEventRecord(e0), "record")) return false;
  hipLaunchKernelGGL(lds_rate_kernel<MODE>, dim3(ncu), dim3(512), 0, 0, cycles, sink);
  if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(e1), "record") || !ok(hipEventSynchronize(e1), "sync"))
    return false;
  float ms = 0.f;
  if (!ok(hipEventElapsedTime(&ms, e0, e1), "elapsed")) return false;
  std::vector<unsigned long long> c(ncu);
  if (!ok(hipMemcpy(c.data(), cycles, ncu * sizeof(unsigned long long), hipMemcpyDeviceToHost), "copy"))
    return false;
  double mean = 0.0;
  for (unsigned long long v : c) mean += (double)v;
  mean /= ncu;
  const double bytes = 8.0 * kIters * 16 * bytes_per_read;  // per workgroup
  std::printf("{\"read\": \"%s\", \"us\": %.1f, \"cycles\": %.0f, \"clock_ghz\": %.3f, \"bytes_per_clk_per_cu\": %.1f}\n",
              name, ms * 1e3, mean, mean / (ms * 1e6), bytes / mean);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return true;
}

}  // namespace

int main() {
  int ncu = 0;
  if (!ok(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0), "attribute")) return 1;
  unsigned long long* cycles = nullptr;
  uint32_t* sink = nullptr;
  if (!ok(hipMalloc(&cycles, ncu * sizeof(unsigned long long)), "malloc") ||
      !ok(hipMalloc(&sink, (size_t)ncu * 512 * sizeof(uint32_t)), "malloc"))
    return 1;
  const bool good = measure<0>(ncu, cycles, sink, "ds_read_b128", 1024) &&
                    measure<1>(ncu, cycles, sink, "ds_read_b64_tr_b16", 512) &&
                    measure<2>(ncu, cycles, sink, "ds_read_b64", 512);
  hipFree(cycles);
  hipFree(sink);
  return good ? 0 : 1;
}
