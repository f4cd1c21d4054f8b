// Device-side building blocks shared by the gfx950 attention kernels: operand types,
// CDNA4 MFMA wrappers, LDS transpose reads, conversions and lane exchanges.
//
// MFMA v_mfma_f32_32x32x16_{bf16,f16} operand layout (lane l of a 64-wide wavefront,
// h = l / 32, i = l % 32; verified on gfx950):
//   A (32 x 16): lane holds A[i][8h .. 8h+7]
//   B (16 x 32): lane holds B[8h .. 8h+7][i]
//   C (32 x 32): lane holds C[8*(r/4) + 4h + (r%4)][i] in register r = 0..15
// ds_read_b64_tr_b16, per group of 16 lanes: lane i receives element (i % 4) of the four
// 8-byte chunks addressed by lanes (i / 4) + 4j, j = 0..3, of its group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

// 8 packed 16-bit values (one MFMA operand) carried type-agnostically.
struct Frag8 {
  u32x4 v;
};

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32x32x16(const Frag8& a, const Frag8& b, const f32x16& c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v), __builtin_bit_cast(bf16x8, b.v), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a.v), __builtin_bit_cast(f16x8, b.v), c, 0,
                                                  0, 0);
  }
}

// Two fp32 -> one dword of two 16-bit values, round-to-nearest-even.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (BF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 t = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, t);
  } else {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 t = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, t);
  }
}

// acc + lo + hi of two packed 16-bit values, in fp32 (one v_dot2 against (1, 1)).
template <bool BF16>
__device__ __forceinline__ float sum2(uint32_t two, float acc) {
  if constexpr (BF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, two), one, acc, false);
  } else {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, two), one, acc, false);
  }
}

template <bool BF16>
__device__ __forceinline__ float to_f32(uint16_t bits) {
  if constexpr (BF16) {
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, bits);
  }
}

// 8-byte transposed LDS read (see the layout note above).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* lds_ptr) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(lds_ptr));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// An int loaded from a wavefront-uniform address, kept in a scalar register.  The compiler
// cannot prove such a load uniform; without this, buffer resources and offsets built from
// the value sit in vector registers and every buffer access becomes a loop over lanes.
__device__ __forceinline__ int load_uniform(const int32_t* p) { return __builtin_amdgcn_readfirstlane(*p); }

// True when the device-side argument checks (FA_DEBUG_CHECKS=1) have flagged an error
// earlier on the stream: the kernel then returns before doing anything.  `flag` is null
// when the checks are off.
__device__ __forceinline__ bool debug_stop(const int* flag) {
  return flag != nullptr && __builtin_amdgcn_readfirstlane(*flag) != 0;
}

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4): lane l of the
// wavefront writes lds_base + 16*l.  lds_base must be the same in every lane.
__device__ __forceinline__ void lds_direct_load16(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (FA_LDS void*)lds_base, 16, 0, 0);
}

// The same load from a wavefront-uniform base plus an unsigned 32-bit per-lane byte
// offset: this is the instruction's scalar-base form, so no per-lane 64-bit address has to
// be formed.
__device__ __forceinline__ void lds_direct_load16(const void* base, uint32_t byte_off, void* lds_base) {
  lds_direct_load16((const char*)base + byte_off, lds_base);
}

// Bytes from element `first` to the end of an array of `total` elements of `esize` bytes,
// clamped to the 32-bit extent of a buffer resource (0 when `first` is past the end).
__device__ __forceinline__ uint32_t bytes_left(size_t total, size_t first, uint32_t esize) {
  if (first >= total) return 0u;
  const size_t b = (total - first) * esize;
  return b < 0xffffffffu ? (uint32_t)b : 0xffffffffu;
}

// Buffer resource for raw (unstructured) buffer loads over [base, base + bytes): offsets
// at or past `bytes` read as zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from buffer offset byte_off + uniform_off straight into LDS
// (buffer_load_dwordx4 with the lds bit; uniform_off goes in the scalar offset and is
// not range-checked): lane l writes lds_base + 16*l.  Unlike the flat-encoded global form, this
// load does not count against the LDS wait counter, so later LDS reads can still be
// waited for one by one.
__device__ __forceinline__ void lds_buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, void* lds_base,
                                                  uint32_t uniform_off = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)lds_base, 16, byte_off, (int)uniform_off, 0, 0);
}

// The same load with the non-temporal (streaming) cache hint, for data read exactly once.
__device__ __forceinline__ void lds_buffer_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)lds_base, 16, byte_off, 0, 0, 2);
}

// The same with 4 bytes per lane (buffer_load_dword with the lds bit): lane l writes
// lds_base + 4*l.
__device__ __forceinline__ void lds_buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)lds_base, 4, byte_off, 0, 0, 0);
}

// 16-byte store per lane at buffer offset byte_off; offsets at or past the resource's
// extent are dropped by the hardware.
__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)byte_off, 0, 0);
}

// 4 bytes per lane straight into LDS (global_load_lds_dword): lane l writes lds_base + 4*l.
__device__ __forceinline__ void lds_direct_load4(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (FA_LDS void*)lds_base, 4, 0, 0);
}

// Wait until every outstanding memory operation of this wavefront has completed
// (including direct global->LDS loads).
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N vector-memory operations of this wavefront are outstanding,
// leaving LDS and export counters alone.  Loads complete in issue order among themselves,
// so with only loads in flight N > 0 means "all but the last N have landed".  Stores and
// atomics share the counter but are not ordered against loads: while any is in flight,
// only N = 0 says which loads have landed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS traffic only: this wavefront's LDS operations are complete
// before it arrives, and the compiler keeps memory accesses on their side of it.  Global
// loads, stores and atomics in flight are not waited for (a __syncthreads() would wait
// for all of them, including direct global->LDS loads); callers that need those wait
// with wait_vmcnt first.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((15 & 15) | (3 << 14) | (7 << 4));  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// Register values that must be complete where the call stands: an empty asm statement
// that reads and rewrites them, so that the compiler cannot sink their computation past a
// phase barrier.
__device__ __forceinline__ void pin(f32x16& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(u32x4& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// Workgroup barrier that also fences the instruction scheduler, so that no product or
// softmax instruction migrates into the neighbouring phase of a ping-pong schedule.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <int I>
using Idx = std::integral_constant<int, I>;

// f(Idx<I>), f(Idx<I+1>), ..., f(Idx<N-1>), unrolled at compile time.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Head dimensions that are not a tile size: a kernel instantiated for tile width D
// (64, 128 or 256) serves any head dimension Dr <= D with Dr % 8 == 0.  Rows in LDS keep D
// elements; the 16-byte chunks past Dr / 8 are padding.  One operand of every product over
// the head dimension holds zeros there (the query side of S in the forward, the key and
// value side in the backward), and the other re-reads chunk 0 of the same row
// (src_chunk), so the padding adds exact zeros and no load leaves the row; products whose
// output columns fall in the padding are never stored.
__device__ __forceinline__ int src_chunk(int g, int dc) { return g < dc ? g : 0; }

// Combine a value with the one held by lane l^32 (the other half of the wavefront).
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// One layout serving both read patterns on the same tile: 16-byte row reads of 16
// consecutive rows (MFMA operands taken along the head dimension) and transposed 8-byte
// reads of 4 consecutive rows x 4 consecutive chunks (operands taken along the rows).
// f(r) is a bijection on 16 consecutive rows whose low two bits of r select the 4-chunk
// group, so both patterns land on 16 distinct 4-bank groups.
template <int D>
struct DualSwizzle {
  static constexpr int CH = D / 8;
  __device__ static __forceinline__ int f(int r) {
    if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return ((r & 3) << 2) | ((r >> 2) & 3);
  }
  __device__ static __forceinline__ int chunk(int r, int c) { return c ^ f(r); }
  __device__ static __forceinline__ int row_elem(int r, int c) { return r * D + chunk(r, c) * 8; }
  __device__ static __forceinline__ int elem(int r, int e) { return r * D + chunk(r, e >> 3) * 8 + (e & 7); }
};

// Returns x unchanged but hides its value from the optimiser, so that expressions built
// from it inside a loop are recomputed there instead of being hoisted into registers
// that stay live across the whole loop (an empty asm statement; emits no instruction).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Kept keys of query row i of a sequence (bottom-right aligned, diag = Lk - Lq): the
// causal limit, the sliding window and the end of the sequence, as a closed range.
struct KeyWindow {
  int Lk, diag, causal, wl, wr;
  __device__ __forceinline__ int lo(int i) const { return wl >= 0 ? (i + diag - wl > 0 ? i + diag - wl : 0) : 0; }
  __device__ __forceinline__ int hi(int i) const {
    int h = Lk - 1;
    if (causal) {
      h = h < i + diag ? h : i + diag;
    } else if (wr >= 0) {
      h = h < i + diag + wr ? h : i + diag + wr;
    }
    return h;
  }
};

__device__ __forceinline__ u32x4 load16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void store16(void* p, u32x4 x) { *(u32x4*)p = x; }

}  // namespace fa
