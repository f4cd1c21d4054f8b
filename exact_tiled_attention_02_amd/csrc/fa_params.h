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
  float* dsum;    // fp32 [rows, Hq]
  const int32_t* cu_q;
  const int32_t* cu_k;
  int B, Sq, Sk, Hq, Hkv, D;
  int causal;
  int bf16;
  float scale;
  float scale_log2;
  int zero_acc;  // preprocess also zeroes dq_acc (the atomic path needs it)
};

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// stage_mask bit 0: preprocess, bit 1: main loop with dQ atomics, bit 2: finalize,
// bit 3: deterministic dQ (main loop without dQ, then a separate dQ pass writing dq).
hipError_t launch_bwd(const BwdArgs& a, int stage_mask, hipStream_t stream);

}  // namespace fa
