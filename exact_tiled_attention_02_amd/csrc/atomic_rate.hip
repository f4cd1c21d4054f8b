// Measurement program (not part of libfa.so): the rate at which MI355X executes fp32 atomic
// adds to device memory in the pattern of the backward's dQ accumulation -- each wavefront
// instruction adds 64 floats (two rows of 32 consecutive columns, or one row of 64) with a
// buffer atomic that returns nothing, all 256 CUs issuing -- and, for comparison, packed
// 16-bit atomic adds.  Prints one JSON line per variant.  The backward main loop adds one
// fp32 dQ value per (query row, head, column, 256-key block), so this rate bounds it from below:
// time >= atomics / rate.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <vector>

namespace {

constexpr int kRows = 8192, kHeads = 16, kD = 128;  // a 64 MiB fp32 accumulator
constexpr int kRowBytes = kHeads * kD * 4;

// Mode 0: the dQ pattern (lanes = 2 rows x 32 columns, 16 instructions per step);
// mode 1: one row of 64 consecutive floats per instruction; mode 2: packed fp16 pairs,
// one row of 128 consecutive halves per instruction (8 instructions per step).
template <int MODE>
__global__ __launch_bounds__(256) void atomic_rate_kernel(float* acc, int steps) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 31, lh = lane >> 5;
  const auto r = __builtin_amdgcn_make_buffer_rsrc(acc, 0, kRows * kRowBytes, 0x00020000);
  for (int s = 0; s < steps; ++s) {
    const int h = (s * 7 + (int)blockIdx.x) & (kHeads - 1);
    const int row0 = (((int)blockIdx.x * 5 + s * 13) & 255) * 32;
    const int base = (row0 * kHeads + h) * kD * 4;
    if constexpr (MODE == 0) {
      const int voff = 4 * lh * kRowBytes + (wave * 32 + li) * 4;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(1.0f, r, base + voff, (8 * (q >> 2) + (q & 3)) * kRowBytes, 0);
    } else if constexpr (MODE == 1) {
      const int voff = ((wave & 1) * 64 + lane) * 4;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(1.0f, r, base + voff, (q * 2 + (wave >> 1)) * kRowBytes, 0);
    } else {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
      for (int q = 0; q < 8; ++q)
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_v2f16(one, r, base + lane * 4, (q * 4 + wave) * kRowBytes, 0);
    }
  }
}

int check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
  }
  return 0;
}

template <int MODE>
int run(float* acc, const char* name, int steps) {
  const size_t bytes = (size_t)kRows * kRowBytes;
  hipEvent_t e0, e1;
  if (check(hipEventCreate(&e0), "event") || check(hipEventCreate(&e1), "event")) return 1;
  hipLaunchKernelGGL(atomic_rate_kernel<MODE>, dim3(256), dim3(256), 0, 0, acc, 4);  // warm-up
  if (check(hipMemset(acc, 0, bytes), "memset") || check(hipDeviceSynchronize(), "sync")) return 1;
  if (check(hipEventRecord(e0), "record")) return 1;
  hipLaunchKernelGGL(atomic_rate_kernel<MODE>, dim3(256), dim3(256), 0, 0, acc, steps);
  if (check(hipEventRecord(e1), "record") || check(hipEventSynchronize(e1), "sync")) return 1;
  float ms = 0.f;
  if (check(hipEventElapsedTime(&ms, e0, e1), "elapsed")) return 1;
  // every element added must be there: sum of the accumulator = number of additions
  std::vector<float> h(bytes / 4);
  if (check(hipMemcpy(h.data(), acc, bytes, hipMemcpyDeviceToHost), "copy")) return 1;
  double sum = 0.0;
  if (MODE == 2) {
    const _Float16* p = reinterpret_cast<const _Float16*>(h.data());
    for (size_t i = 0; i < h.size() * 2; ++i) sum += (double)(float)p[i];
  } else {
    for (float x : h) sum += x;
  }
  const double adds = 256.0 * 4 * 16 * 64 * steps;  // per launch: 256 workgroups x 4 waves x 1024 values
  printf("{\"variant\": \"%s\", \"us\": %.1f, \"adds_per_s\": %.4g, \"requests_64B_per_s\": %.4g, "
         "\"sum_over_expected\": %.6f}\n",
         name, ms * 1e3, adds / (ms * 1e-3), adds / (MODE == 2 ? 32.0 : 16.0) / (ms * 1e-3), sum / adds);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return 0;
}

}  // namespace

int main() {
  float* acc = nullptr;
  if (check(hipMalloc(&acc, (size_t)kRows * kRowBytes), "malloc")) return 1;
  int rc = run<0>(acc, "fp32, 2 rows x 32 columns per instruction (dQ pattern)", 256);
  rc |= run<1>(acc, "fp32, 1 row x 64 columns per instruction", 256);
  rc |= run<2>(acc, "packed fp16 pairs, 1 row x 128 halves per instruction", 256);
  hipFree(acc);
  return rc;
}
