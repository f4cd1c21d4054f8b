// Backward kernels: preprocess, dK/dV main loop with dQ accumulation, dQ finalize.
//
// The probabilities are recomputed from the forward's LSE instead of being stored: the
// backward of the release notes "v1.4 - FlashAttention Fork" (section 4.1) applies
// exp2 with the stored per-row value multiplied by log2(e), i.e.
// P = exp2(S * scale*log2(e) - LSE * log2(e)).  With that P the gradients are the
// analytic ones of O = softmax(scale Q K^T) V:
//   dV = P^T dO,  dP = dO V^T,  Dsum_i = sum_d dO_id O_id,  dS = P * (dP - Dsum),
//   dK = scale dS^T Q,  dQ = scale dS K.
// dK/dV of a KV head sum over the query heads that share it (MQA/GQA rule of the
// flash_attn_func docstring); the causal mask is bottom-right aligned as in the forward.
//
// Kernels (all on the caller's stream, in order):
//   1. preprocess: -Dsum = -rowsum(dO * O) in fp32 (the D <= 128 main loop starts dP from
//      it), LSE * log2(e), and zeroing of the fp32 dQ accumulator (memory-bound);
//   2. main loop, one workgroup per (key block, KV head, sequence), walking the query
//      blocks that can see its keys for every query head of the group, so dK and dV
//      accumulate in registers with no atomics.  Per query step: S = Q K^T, P,
//      dP = dO V^T, dS, then dV^T += dO^T P and dK^T += Q^T dS on MFMA; dS goes through
//      LDS so that the workgroup forms dQ = dS K for the step's rows over all its keys,
//      added to the fp32 accumulator with atomics.  Head dimensions up to 128 use 256
//      keys per workgroup (8 wavefronts of 32 keys); D = 256 uses 128 keys (4
//      wavefronts), which its register footprint requires;
//   3. finalize: scale * fp32 accumulator -> dQ in the input dtype.
// Two routes form dQ without atomics.  The stored-dS route (fa_bwd's when the workspace
// holds the area): the main loop without the dQ product stores each step's dS / scale in
// the input dtype -- the values the dQ product would have taken -- and a memory-bound pass
// (2d) forms dQ = scale dS K once per query row from them.  The recompute route (2c, no
// extra workspace): a forward-shaped pass computes S and dP a second time.
// The main loops form dS / scale (one multiply less per score) and apply the softmax scale
// once to dK at its store and to dQ in the finalize or the dQ passes; the preprocess also
// writes LSE * log2(e) per (row, head), the exp2 offset of P in the D <= 128 main loop.
// Sliding window and ALiBi (flash_attn_func docstring, window_size and alibi_slopes): the
// kept keys of query i are [lo(i), hi(i)] as in the forward (KeyWindow); the main loops
// visit only the query rows that keep a key of their block, and the ALiBi bias
// -slope * |i + Lk - Lq - j| enters P through the exponent (it does not depend on q, k or
// v, so the gradient formulas are unchanged).
#include <type_traits>

#include <algorithm>

#include "fa_device.h"
#include "fa_params.h"

namespace fa {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdBN = 32 * kBwdWaves;  // keys per workgroup
constexpr int kBwdBQ = 32;              // query rows per inner step

// Query steps (32-row blocks of a sequence) that keep a key of the key block
// [k0, k0 + nkeys): [begin, end), empty when begin == end.  Bottom-right causal limit and
// sliding window as in KeyWindow; without a mask every row keeps every key.  The main loops
// visit exactly these steps, and the dQ pass over stored dS reads exactly the tiles they
// wrote, so both take the range from here.
struct StepRange {
  int begin, end;
};
__device__ __forceinline__ StepRange block_steps(int k0, int nkeys, int Lq, int Lk, bool masked, int causal, int wl,
                                                 int wr) {
  const int diag = Lk - Lq;
  const int k_last = min(k0 + nkeys, Lk) - 1;
  int i_begin = 0, i_end = Lq;
  if (masked) {
    if (causal) {
      i_begin = max(0, k0 - diag);
    } else if (wr >= 0) {
      i_begin = max(0, k0 - diag - wr);
    }
    if (wl >= 0) i_end = min(Lq, k_last - diag + wl + 1);
  }
  const int qb = i_begin / 32;
  return StepRange{qb, i_end > i_begin ? (i_end + 31) / 32 : qb};
}

// ---------------------------------------------------------------- 1. preprocess

template <int D, bool BF16, bool VARLEN>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  if (debug_stop(a.dbg)) return;
  constexpr int CH = D / 8;              // 16-byte chunks per (row, head)
  constexpr int PAIRS = 256 / CH;        // (row, head) pairs per workgroup
  const int tid = threadIdx.x;
  const int pair_local = tid / CH;
  const int ch = tid % CH;
  const size_t pair = (size_t)blockIdx.x * PAIRS + pair_local;
  size_t rows = (size_t)a.B * a.Sq;  // the workspace's rows (a bound on total_q)
  if constexpr (VARLEN) rows = min(rows, (size_t)max(load_uniform(a.cu_q + a.B), 0));
  const bool live = pair < rows * a.Hq;
  float s = 0.f;
  if (live && ch * 8 < a.D) {  // lanes past the head dimension add nothing
    const size_t off = pair * a.D + ch * 8;
    const u32x4 o = load16((const uint16_t*)a.out + off);
    const u32x4 g = load16((const uint16_t*)a.dout + off);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s += to_f32<BF16>(o[w] & 0xffff) * to_f32<BF16>(g[w] & 0xffff);
      s += to_f32<BF16>(o[w] >> 16) * to_f32<BF16>(g[w] >> 16);
    }
    if (a.zero_acc) {
      float* acc = a.dq_acc + off;
      store16(acc, u32x4{0, 0, 0, 0});
      store16(acc + 4, u32x4{0, 0, 0, 0});
    }
  }
  // reduce over the CH lanes of this pair (CH is a power of two <= 32, lanes contiguous)
#pragma unroll
  for (int m = CH / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (live && ch == 0) {
    a.dsum[pair] = -s;  // stored negated: the D <= 128 main loop starts dP from it
    // LSE * log2(e) in the same [row, head] layout (the exp2 offset the main loop needs)
    const size_t row = pair / a.Hq;
    const int h = (int)(pair % a.Hq);
    size_t li;
    if constexpr (VARLEN) {
      li = (size_t)h * rows + row;  // lse [Hq, total_q]
    } else {
      li = ((row / a.Sq) * a.Hq + h) * a.Sq + row % a.Sq;  // lse [B, Hq, Sq]
    }
    a.lse2[pair] = a.lse[li] * 1.4426950408889634f;
  }
  if (blockIdx.x == 0 && tid == 0) {  // the main loop's key-block queue starts empty
    a.work[0] = 0;
    a.work[1] = 0;
  }
}

// ---------------------------------------------------------------- 2a. main loop, D = 256

template <int D, bool BF16, bool MASKED, bool VARLEN, bool DQ, bool ALIBI>
__global__ __launch_bounds__(256) void bwd_main_kernel(BwdArgs a) {
  if (debug_stop(a.dbg)) return;
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int SSTR = kBwdBN + 8;  // dS tile [query row][key], padded
  constexpr int QT = kBwdBQ * D;    // elements of a Q or dO tile
  using Swz = DualSwizzle<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBwdBN * D];
  // Step buffers as distinct LDS objects (double-buffered by step), so that the compiler
  // can tell the reads of one step from the direct loads in flight into the other.
  __shared__ __attribute__((aligned(16))) uint16_t Q0[QT];
  __shared__ __attribute__((aligned(16))) uint16_t Q1[QT];
  __shared__ __attribute__((aligned(16))) uint16_t dO0[QT];
  __shared__ __attribute__((aligned(16))) uint16_t dO1[QT];
  __shared__ __attribute__((aligned(16))) uint16_t dSs[kBwdBQ * SSTR];
  __shared__ __attribute__((aligned(16))) float lse0[64];
  __shared__ __attribute__((aligned(16))) float lse1[64];
  __shared__ __attribute__((aligned(16))) float dsum0[64];
  __shared__ __attribute__((aligned(16))) float dsum1[64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int lh = lane >> 5;

  const int nbh = a.B * a.Hkv;
  const int kb = blockIdx.x / nbh;
  const int bh = blockIdx.x % nbh;
  const int hk = bh % a.Hkv;
  const int b = bh / a.Hkv;

  int q_start, k_start, Lq, Lk;
  if constexpr (VARLEN) {
    q_start = load_uniform(a.cu_q + b);
    Lq = load_uniform(a.cu_q + b + 1) - q_start;
    k_start = load_uniform(a.cu_k + b);
    Lk = load_uniform(a.cu_k + b + 1) - k_start;
  } else {
    q_start = b * a.Sq;
    Lq = a.Sq;
    k_start = b * a.Sk;
    Lk = a.Sk;
  }
  const int k0 = kb * kBwdBN;
  if (k0 >= Lk) return;  // uniform

  const int G = a.Hq / a.Hkv;
  const int Dr = a.D;  // head dimension of the tensors (<= D, the tile width)
  const int Dc = Dr / 8;
  const size_t q_rs = (size_t)a.Hq * Dr;
  const size_t k_rs = (size_t)a.Hkv * Dr;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)k_start * k_rs + (size_t)hk * Dr;
  const uint16_t* vp = (const uint16_t*)a.v + (size_t)k_start * k_rs + (size_t)hk * Dr;
  const int diag = Lk - Lq;
  const float c = a.scale_log2;
  const float inv_c = 1.0f / c;  // (as in the main loop for D <= 128)
  constexpr float kLog2e = 1.4426950408889634f;
  size_t lse_row0;  // index of row 0 of this sequence in the LSE of head 0
  size_t lse_hs;    // LSE stride between heads
  if constexpr (VARLEN) {
    lse_hs = (size_t)load_uniform(a.cu_q + a.B);
    lse_row0 = (size_t)q_start;
  } else {
    lse_hs = (size_t)a.Sq;
    lse_row0 = (size_t)b * a.Hq * a.Sq;
  }

  // The work is the flat list of (query head of the group, 32-row query block) steps over
  // the query blocks that keep a key of this block.
  int rmin = -0x3fffffff, rmax = 0x3fffffff;  // rows that keep this lane's key
  const int my_key = k0 + threadIdx.x / 64 * 32 + (threadIdx.x & 31);
  if constexpr (MASKED) {
    if (a.causal) {
      rmin = my_key - diag;
    } else if (a.window_right >= 0) {
      rmin = my_key - diag - a.window_right;
    }
    if (a.window_left >= 0) rmax = my_key - diag + a.window_left;
  }
  const StepRange sr = block_steps(k0, kBwdBN, Lq, Lk, MASKED, a.causal, a.window_left, a.window_right);
  const int qb_begin = sr.begin;
  const int qb_end = sr.end;
  const int nqs = max(0, qb_end - qb_begin);
  const int nsteps = G * nqs;
  float sl_next = 0.f;  // ALiBi slope (exp2 units) of the step fetched last

  // Extents of the arrays the fetch addresses: q / dout hold total_q rows (B * Sq when
  // padded), the LSE Hq * total_q (B * Hq * Sq) values, Dsum B * Sq rows of Hq.
  const size_t q_rows = VARLEN ? (size_t)load_uniform(a.cu_q + a.B) : (size_t)a.B * a.Sq;
  const size_t lse_total = VARLEN ? (size_t)a.Hq * q_rows : (size_t)a.B * a.Hq * a.Sq;
  const size_t ws_rows = (size_t)a.B * a.Sq;

  // Direct global->LDS fetch of step it's Q, dO tiles and per-row LSE, Dsum, in the buffer
  // form (the flat form would make the compiler wait for every LDS read of the loop with
  // lgkmcnt(0)).  Rows past the end of the sequence re-read its last row (they are masked
  // to P = 0).
  auto fetch = [&](int it, uint16_t* __restrict__ Qd, uint16_t* __restrict__ dOd, float* __restrict__ lsed,
                   float* __restrict__ dsumd) {
    const int g = it / nqs;
    const int h = hk * G + g;
    const int i0 = (qb_begin + it % nqs) * kBwdBQ;
    const size_t base = (size_t)(q_start + i0) * q_rs + (size_t)h * Dr;
    const uint32_t qbytes = bytes_left(q_rows * q_rs, base, 2u);
    const auto qr = make_rsrc((const uint16_t*)a.q + base, qbytes);
    const auto gr = make_rsrc((const uint16_t*)a.dout + base, qbytes);
#pragma unroll
    for (int i = 0; i < QT / 8 / 256; ++i) {
      const int first = (i * kBwdWaves + wave) * 64;
      const int chunk = first + lane;
      const int r = chunk / Swz::CH;
      const int p = chunk % Swz::CH;
      const uint32_t src = (uint32_t)(min(r, Lq - 1 - i0) * (int)q_rs + src_chunk(Swz::chunk(r, p), Dc) * 8) * 2u;
      lds_buffer_load16(qr, src, Qd + first * 8);
      lds_buffer_load16(gr, src, dOd + first * 8);
    }
    const uint32_t rr = (uint32_t)(min(i0 + (lane & 31), Lq - 1) - i0);
    if (wave == 0) {
      const size_t lbase = lse_row0 + (size_t)h * lse_hs + i0;
      lds_buffer_load4(make_rsrc(a.lse + lbase, bytes_left(lse_total, lbase, 4u)), rr * 4u, lsed);
    }
    if (wave == 1) {
      const size_t dbase = (size_t)(q_start + i0) * a.Hq + h;
      lds_buffer_load4(make_rsrc(a.dsum + dbase, bytes_left(ws_rows * a.Hq, dbase, 4u)), rr * (uint32_t)a.Hq * 4u,
                       dsumd);
    }
    if constexpr (ALIBI) sl_next = a.alibi[(size_t)b * a.alibi_bstride + h] * kLog2e;
  };

  if (nsteps > 0) fetch(0, Q0, dO0, lse0, dsum0);
  // K tile (all 128 keys, rows clamped to the sequence) in LDS, for S = Q K^T (row reads)
  // and dQ = dS K (transposed reads), by buffer loads from the block's first key; chunks
  // past the head dimension get an offset beyond the resource's extent and read as zeros
  // (lane offsets of real chunks stay below 128 rows * Hkv * D * 2 < 2^31 bytes).
  {
    const size_t kfirst = (size_t)(k_start + k0) * k_rs + (size_t)hk * Dr;
    const size_t k_rows = VARLEN ? (size_t)load_uniform(a.cu_k + a.B) : (size_t)a.B * a.Sk;
    const auto kr = make_rsrc((const uint16_t*)a.k + kfirst, min(bytes_left(k_rows * k_rs, kfirst, 2u), 0x7fffffffu));
#pragma unroll
    for (int i = 0; i < kBwdBN * D / 8 / 256; ++i) {
      const int first = (i * kBwdWaves + wave) * 64;
      const int chunk = first + lane;
      const int r = chunk / Swz::CH;
      const int g = Swz::chunk(r, chunk % Swz::CH);
      const uint32_t off = g < Dc ? (uint32_t)(min(r, Lk - 1 - k0) * (int)k_rs + g * 8) * 2u : 0x80000000u;
      lds_buffer_load16(kr, off, &Ks[first * 8]);
    }
  }

  // This wavefront's values as B operands of dP = dO V^T: lane holds V[key][16 s + 8 lh ..
  // +7], zero past the head dimension (the padded Q / dO chunks re-read chunk 0).  Its
  // keys for S come from the K tile in LDS (registers for both would not fit beside the
  // 256 accumulators of dK and dV).
  const bool key_ok = my_key < Lk;
  Frag8 vf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    vf[s].v = key_ok && s * 16 + lh * 8 < Dr ? load16(vp + (size_t)my_key * k_rs + s * 16 + lh * 8)
                                             : u32x4{0, 0, 0, 0};
  f32x16 dkt[ND], dvt[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    dkt[d] = f32x16{};
    dvt[d] = f32x16{};
  }

  const int tr_row = 4 * lh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  wait_all_memory();
  __syncthreads();

  auto step = [&](int it, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ dO,
                  const float* __restrict__ lse_c, const float* __restrict__ dsum_c, uint16_t* __restrict__ Qn,
                  uint16_t* __restrict__ dOn, float* __restrict__ lse_n, float* __restrict__ dsum_n) {
    const int h = hk * G + it / nqs;
    const int i0 = (qb_begin + it % nqs) * kBwdBQ;
    const float sl = sl_next;
    if (it + 1 < nsteps) fetch(it + 1, Qn, dOn, lse_n, dsum_n);

    // S = Q K^T and dP = dO V^T (query rows x keys); lane = key, registers = rows.  The
    // row reads run RA k-steps ahead of their products, in fenced order (left to itself
    // the scheduler sinks each read down to its product); with the dQ product (the staged
    // atomic route) one step ahead, as more registers would spill.
    // The accumulators start from -LSE log2(e) / c and -Dsum (register r = 4 g4 + j holds
    // row 8 g4 + 4 lh + j; both come as vectors), so that the products leave S - LSE / scale
    // and dP - Dsum, and no LSE or Dsum read waits after them.
    f32x16 s, dp;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 l4 = *(const f32x4*)(lse_c + 8 * g4 + 4 * lh);
      const f32x4 d4 = *(const f32x4*)(dsum_c + 8 * g4 + 4 * lh);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[4 * g4 + j] = -l4[j] * (kLog2e * inv_c);
        dp[4 * g4 + j] = d4[j];
      }
    }
    {
      constexpr int RA = DQ ? 1 : 2;
      Frag8 qa[RA], ga[RA], kf[RA];
      auto issue = [&](auto st_tag) __attribute__((always_inline)) {
        constexpr int st = decltype(st_tag)::value, sl2 = st % RA;
        const int off = Swz::row_elem(li, st * 2 + lh);
        qa[sl2].v = load16(Q + off);
        ga[sl2].v = load16(dO + off);
        kf[sl2].v = load16(Ks + wave * 32 * D + off);  // key row wave*32 + li: the same swizzle as row li
      };
      static_for<0, RA>([&](auto st) __attribute__((always_inline)) { issue(st); });
      static_for<0, NS>([&](auto st_tag) __attribute__((always_inline)) {
        constexpr int st = decltype(st_tag)::value, sl2 = st % RA;
        __builtin_amdgcn_sched_barrier(0);
        s = mfma32x32x16<BF16>(qa[sl2], kf[sl2], s);
        dp = mfma32x32x16<BF16>(ga[sl2], vf[st], dp);
        if constexpr (st + RA < NS) issue(Idx<st + RA>{});
      });
      __builtin_amdgcn_sched_barrier(0);
    }
    // P and dS / scale (the scale is applied to dK at its store and to dQ in the finalize).
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * g4 + j;
        const int row = i0 + 8 * g4 + 4 * lh + j;
        bool keep = key_ok && row < Lq;
        if constexpr (MASKED) keep = keep && row >= rmin && row <= rmax;
        float e = s[r] * c;
        if constexpr (ALIBI) e = fmaf(s[r], c, -sl * fabsf((float)(row + diag - my_key)));
        const float p = keep ? fast_exp2(e) : 0.f;
        s[r] = p;
        dp[r] = p * dp[r];  // dS / scale = P (dP - Dsum)
      }
    }
    Frag8 pf[2], dsf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r0 = 8 * t;
      pf[t].v = u32x4{pack2<BF16>(s[r0 + 0], s[r0 + 1]), pack2<BF16>(s[r0 + 2], s[r0 + 3]),
                      pack2<BF16>(s[r0 + 4], s[r0 + 5]), pack2<BF16>(s[r0 + 6], s[r0 + 7])};
      dsf[t].v = u32x4{pack2<BF16>(dp[r0 + 0], dp[r0 + 1]), pack2<BF16>(dp[r0 + 2], dp[r0 + 3]),
                       pack2<BF16>(dp[r0 + 4], dp[r0 + 5]), pack2<BF16>(dp[r0 + 6], dp[r0 + 7])};
    }
    // dS to LDS as [row][key] for the dQ product.
#pragma unroll
    for (int t = 0; t < (DQ ? 2 : 0); ++t) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t two = dsf[t].v[w];
        const int r = 8 * t + 2 * w;  // registers r and r+1 of this lane
        const int rl0 = 8 * (r >> 2) + 4 * lh + (r & 3);
        dSs[rl0 * SSTR + wave * 32 + li] = (uint16_t)(two & 0xffff);
        dSs[(rl0 + 1) * SSTR + wave * 32 + li] = (uint16_t)(two >> 16);
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS over ops (t, d), transposed reads RA ops ahead.
    {
      constexpr int RA = DQ ? 1 : 2, NO = 2 * ND;
      Frag8 ga[RA], qa[RA];
      auto issue = [&](auto o_tag) __attribute__((always_inline)) {
        constexpr int o = decltype(o_tag)::value, sl2 = o % RA, t = o / ND, d = o % ND;
        const int row = t * 16 + tr_row;
        const int col = d * 32 + tr_col;
        const int o_lo = Swz::elem(row, col), o_hi = Swz::elem(row + 8, col);
        const u32x2 g_lo = lds_read_tr16(dO + o_lo);
        const u32x2 g_hi = lds_read_tr16(dO + o_hi);
        const u32x2 q_lo = lds_read_tr16(Q + o_lo);
        const u32x2 q_hi = lds_read_tr16(Q + o_hi);
        ga[sl2].v = u32x4{g_lo.x, g_lo.y, g_hi.x, g_hi.y};
        qa[sl2].v = u32x4{q_lo.x, q_lo.y, q_hi.x, q_hi.y};
      };
      static_for<0, RA>([&](auto o) __attribute__((always_inline)) { issue(o); });
      static_for<0, NO>([&](auto o_tag) __attribute__((always_inline)) {
        constexpr int o = decltype(o_tag)::value, sl2 = o % RA, t = o / ND, d = o % ND;
        __builtin_amdgcn_sched_barrier(0);
        dvt[d] = mfma32x32x16<BF16>(ga[sl2], pf[t], dvt[d]);
        dkt[d] = mfma32x32x16<BF16>(qa[sl2], dsf[t], dkt[d]);
        if constexpr (o + RA < NO) issue(Idx<o + RA>{});
      });
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (DQ) __syncthreads();  // dS of all four wavefronts is in LDS

    // dQ[rows][d-block] = dS[rows][128 keys] K[128 keys][d-block]; d-blocks are dealt
    // round-robin to the wavefronts.
    for (int d = wave; DQ && d < ND; d += kBwdWaves) {
      f32x16 dq = f32x16{};
#pragma unroll
      for (int ks = 0; ks < kBwdBN / 16; ++ks) {
        Frag8 sa, kb2;
        sa.v = load16(&dSs[li * SSTR + ks * 16 + lh * 8]);
        const int krow = ks * 16 + 8 * lh + ((lane & 15) >> 2);
        const int kcol = d * 32 + tr_col;
        const u32x2 lo = lds_read_tr16(&Ks[Swz::elem(krow, kcol)]);
        const u32x2 hi = lds_read_tr16(&Ks[Swz::elem(krow + 4, kcol)]);
        kb2.v = u32x4{lo.x, lo.y, hi.x, hi.y};
        dq = mfma32x32x16<BF16>(sa, kb2, dq);
      }
      // lane = column d*32 + li; registers = rows.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row < Lq && (size_t)(q_start + row) < (size_t)a.B * a.Sq && d * 32 + li < Dr) {  // inside the accumulator
          float* dst = a.dq_acc + ((size_t)(q_start + row) * a.Hq + h) * Dr + d * 32 + li;
          unsafeAtomicAdd(dst, dq[r]);
        }
      }
    }
    wait_all_memory();  // the prefetched step has landed in LDS
    __syncthreads();    // every wavefront is done with this step's tiles and dS
    if constexpr (!DQ) {
      // As in the main loop for D <= 128: dS / scale of this wavefront's 32 keys x 32 rows
      // into the step's stored tile, when the route over stored dS asks for it (after the
      // wait, so that the stores have a whole step to complete).
      if (a.ds != nullptr && i0 / kBwdBQ < a.ds_nqs) {  // (the step bound fails only for invalid cu_seqlens)
        uint16_t* t = a.ds + (((size_t)b * a.Hq + h) * a.ds_nqs + (size_t)(i0 / kBwdBQ)) * a.ds_nkb * (kBwdBQ * kBwdBN) +
                      (size_t)kb * (kBwdBQ * kBwdBN) + wave * 1024 + li * 32 + lh * 16;
        store16(t, dsf[0].v);
        store16(t + 8, dsf[1].v);
      }
    }
  };
  for (int it = 0; it < nsteps; ++it) {
    const bool odd = it & 1;
    step(it, odd ? Q1 : Q0, odd ? dO1 : dO0, odd ? lse1 : lse0, odd ? dsum1 : dsum0, odd ? Q0 : Q1, odd ? dO0 : dO1,
         odd ? lse0 : lse1, odd ? dsum0 : dsum1);
  }

  // dK, dV: lane = key, registers = head-dimension entries.
  if (key_ok) {
    uint16_t* dkp = (uint16_t*)a.dk + (size_t)(k_start + my_key) * k_rs + (size_t)hk * Dr;
    uint16_t* dvp = (uint16_t*)a.dv + (size_t)(k_start + my_key) * k_rs + (size_t)hk * Dr;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int col = d * 32 + 8 * gq + 4 * lh;
        u32x2 wk, wv;
        wk.x = pack2<BF16>(dkt[d][4 * gq + 0] * a.scale, dkt[d][4 * gq + 1] * a.scale);
        wk.y = pack2<BF16>(dkt[d][4 * gq + 2] * a.scale, dkt[d][4 * gq + 3] * a.scale);
        wv.x = pack2<BF16>(dvt[d][4 * gq + 0], dvt[d][4 * gq + 1]);
        wv.y = pack2<BF16>(dvt[d][4 * gq + 2], dvt[d][4 * gq + 3]);
        if (col < Dr) {  // four columns, all inside or all past the head dimension
          *(u32x2*)(dkp + col) = wk;
          *(u32x2*)(dvp + col) = wv;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- 2b. main loop, D <= 128

// Head dimensions up to 128, 256 keys per workgroup: each dQ element then receives one
// fp32 atomic per 256 keys.  The atomics execute at the memory side and bound the loop,
// so halving them matters more than anything else here.  Eight wavefronts each own 32
// keys for all 32 rows of a query step: S^T/dP and the dV, dK updates are per wavefront;
// the four dQ tiles of a step (32 rows x 32 columns, contracted over all 256 keys) go to
// wavefronts 0..ND-1, one per SIMD, so every SIMD carries the same MFMA load.  V stays in
// registers as MFMA operands; K is in LDS (row reads for S, transposed reads for dQ).
constexpr int kK2Keys = 256;
constexpr int kK2Waves = 8;
constexpr int kK2BQ = 32;
static_assert(kK2BQ == 32 && kBwdBQ == 32, "block_steps counts 32-row query steps");
static_assert(kK2Keys == bwd_block_keys(128) && kBwdBN == bwd_block_keys(256), "stored dS tile sizes");

template <int D, bool BF16, bool MASKED, bool VARLEN, bool DQ, bool ALIBI>
__device__ __forceinline__ void bwd_k256_block(const BwdArgs& a, const int lin) {
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int SSTR = kK2Keys + 8;  // dS tile [query row][key], padded
  constexpr int QT = kK2BQ * D;      // elements of a Q or dO tile
  using Swz = DualSwizzle<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kK2Keys * D];
  __shared__ __attribute__((aligned(16))) uint16_t Q0[QT];
  __shared__ __attribute__((aligned(16))) uint16_t Q1[QT];
  __shared__ __attribute__((aligned(16))) uint16_t dO0[QT];
  __shared__ __attribute__((aligned(16))) uint16_t dO1[QT];
  __shared__ __attribute__((aligned(16))) uint16_t dS0[kK2BQ * SSTR];  // dS, double-buffered by step
  __shared__ __attribute__((aligned(16))) uint16_t dS1[kK2BQ * SSTR];
  __shared__ __attribute__((aligned(16))) float lse0[64];
  __shared__ __attribute__((aligned(16))) float lse1[64];
  __shared__ __attribute__((aligned(16))) float dsum0[64];
  __shared__ __attribute__((aligned(16))) float dsum1[64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int lh = lane >> 5;

  const int nbh = a.B * a.Hkv;
  const int kb = lin / nbh;
  const int bh = lin % nbh;
  const int hk = bh % a.Hkv;
  const int b = bh / a.Hkv;

  int q_start, k_start, Lq, Lk;
  if constexpr (VARLEN) {
    q_start = load_uniform(a.cu_q + b);
    Lq = load_uniform(a.cu_q + b + 1) - q_start;
    k_start = load_uniform(a.cu_k + b);
    Lk = load_uniform(a.cu_k + b + 1) - k_start;
  } else {
    q_start = b * a.Sq;
    Lq = a.Sq;
    k_start = b * a.Sk;
    Lk = a.Sk;
  }
  const int k0 = kb * kK2Keys;
  if (k0 >= Lk) return;  // uniform

  const int G = a.Hq / a.Hkv;
  const int Dr = a.D;  // head dimension of the tensors (<= D, the tile width)
  const int Dc = Dr / 8;
  const size_t q_rs = (size_t)a.Hq * Dr;
  const size_t k_rs = (size_t)a.Hkv * Dr;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)k_start * k_rs + (size_t)hk * Dr;
  const uint16_t* vp = (const uint16_t*)a.v + (size_t)k_start * k_rs + (size_t)hk * Dr;
  const int diag = Lk - Lq;
  const float c = a.scale_log2;
  // 1 / c: the S accumulator starts from -LSE log2(e) / c = -LSE / scale.  c >= 1e-30 (host
  // clamp), and LSE / scale <= max q.k + ln(keys) / scale stays far inside the fp32 range;
  // the exponent c S then carries an absolute error of about 2^-24 |LSE log2(e)|, far
  // below the 16-bit rounding of P.  (A dead row's LSE of +inf gives -inf, and P = 0.)
  const float inv_c = 1.0f / c;
  constexpr float kLog2e = 1.4426950408889634f;

  // Query rows that keep a key of this block, [i_begin, i_end), and the kept range of
  // each row (KeyWindow; without a mask every row keeps [0, Lk - 1]).
  KeyWindow kw{Lk, diag, 0, -1, -1};
  if constexpr (MASKED) kw = KeyWindow{Lk, diag, a.causal, a.window_left, a.window_right};
  const int k_last = min(k0 + kK2Keys, Lk) - 1;
  const StepRange sr = block_steps(k0, kK2Keys, Lq, Lk, MASKED, a.causal, a.window_left, a.window_right);
  const int qb_begin = sr.begin;
  const int qb_end = sr.end;
  const int nqs = max(0, qb_end - qb_begin);
  const int nsteps = G * nqs;
  float sl_next = 0.f;  // ALiBi slope (exp2 units) of the step fetched last

  // Extents of the arrays the buffer resources below address: q / dout hold total_q rows
  // (B * Sq when padded), the workspace arrays B * Sq rows (a bound on total_q).  Every
  // lane offset stays inside them for valid cu_seqlens; with invalid ones the hardware
  // range check drops what falls outside instead of touching other memory.
  const size_t q_rows = VARLEN ? (size_t)load_uniform(a.cu_q + a.B) : (size_t)a.B * a.Sq;
  const size_t ws_rows = (size_t)a.B * a.Sq;

  // Q / dO tile: QT/8 chunks, one direct load per lane for D = 128 (half the lanes
  // for D = 64).
  constexpr int QCH = QT / 8;
  static_assert(QCH <= kK2Waves * 64 && QCH % 64 == 0, "one direct load per lane at most");
  const int qchunk = wave * 64 + lane;
  const bool qloader = wave * 64 < QCH;  // uniform per wavefront
  const int qr = qchunk / Swz::CH;
  // global chunk of this lane's LDS chunk, and its byte offset from the tile's first row
  const uint32_t qoff = (uint32_t)(qr * (int)q_rs + src_chunk(Swz::chunk(qr, qchunk % Swz::CH), Dc) * 8) * 2u;
  // Steps walk (query head of the group, query block) with the block fastest; the
  // position is carried as counters (no division by the runtime block count).
  auto fetch = [&](int h, int i0, uint16_t* __restrict__ Qd, uint16_t* __restrict__ dOd, float* __restrict__ lsed,
                   float* __restrict__ dsumd) {
    // Buffer-form direct loads from the step's first row (the flat form would make the
    // compiler wait for every LDS read with lgkmcnt(0)).  The lane offsets address clamped
    // rows of the sequence.
    const size_t base = (size_t)(q_start + i0) * q_rs + (size_t)h * Dr;
    if (qloader) {
      uint32_t off = qoff;
      if (i0 + kK2BQ > Lq) {
        // rows clamped to the sequence; recomputed from the lane id rather than kept live
        const int qc = opaque(qchunk), r = qc / Swz::CH;
        off = (uint32_t)(min(r, Lq - 1 - i0) * (int)q_rs + src_chunk(Swz::chunk(r, qc % Swz::CH), Dc) * 8) * 2u;
      }
      const uint32_t qbytes = bytes_left(q_rows * q_rs, base, 2u);
      lds_buffer_load16(make_rsrc((const uint16_t*)a.q + base, qbytes), off, Qd + wave * 64 * 8);
      lds_buffer_load16(make_rsrc((const uint16_t*)a.dout + base, qbytes), off, dOd + wave * 64 * 8);
    }
    const uint32_t rr = (uint32_t)min(lane & 31, Lq - 1 - i0);
    const size_t sbase = (size_t)(q_start + i0) * a.Hq + h;
    const uint32_t sbytes = bytes_left(ws_rows * a.Hq, sbase, 4u);
    if (wave == kK2Waves - 1) lds_buffer_load4(make_rsrc(a.lse2 + sbase, sbytes), rr * (uint32_t)a.Hq * 4u, lsed);
    if (wave == kK2Waves - 2) lds_buffer_load4(make_rsrc(a.dsum + sbase, sbytes), rr * (uint32_t)a.Hq * 4u, dsumd);
    // Issued before the step's dQ atomics, so the end-of-step vmcnt wait covers it too.
    if constexpr (ALIBI) sl_next = a.alibi[(size_t)b * a.alibi_bstride + h] * kLog2e;
  };

  if (nsteps > 0) fetch(hk * G, qb_begin * kK2BQ, Q0, dO0, lse0, dsum0);
  // The block's K tile (rows clamped to the sequence) by buffer loads from its first key.
  // Chunks past the head dimension get an offset beyond the resource's extent, which the
  // hardware reads as zeros: K is the zero side of S = Q K^T for a padded head dimension.
  // (Lane offsets of real chunks stay below 256 rows * Hkv * D * 2 < 2^31 bytes, checked
  // by the host.)
  {
    const size_t kfirst = (size_t)(k_start + k0) * k_rs + (size_t)hk * Dr;
    const size_t k_rows = VARLEN ? (size_t)load_uniform(a.cu_k + a.B) : (size_t)a.B * a.Sk;
    const auto kr = make_rsrc((const uint16_t*)a.k + kfirst, min(bytes_left(k_rows * k_rs, kfirst, 2u), 0x7fffffffu));
#pragma unroll
    for (int i = 0; i < kK2Keys * D / 8 / 512; ++i) {
      const int first = (i * kK2Waves + wave) * 64;
      const int chunk = first + lane;
      const int r = chunk / Swz::CH;
      const int g = Swz::chunk(r, chunk % Swz::CH);
      const uint32_t off = g < Dc ? (uint32_t)(min(r, Lk - 1 - k0) * (int)k_rs + g * 8) * 2u : 0x80000000u;
      lds_buffer_load16(kr, off, Ks + first * 8);
    }
  }

  // This wavefront's keys; V as B operands of dP = dO V^T.
  const int my_key = k0 + wave * 32 + li;
  const bool key_ok = my_key < Lk;
  int rmin = -0x3fffffff, rmax = 0x3fffffff;  // query rows that keep my_key
  if constexpr (MASKED) {
    if (a.causal) {
      rmin = my_key - diag;
    } else if (a.window_right >= 0) {
      rmin = my_key - diag - a.window_right;
    }
    if (a.window_left >= 0) rmax = my_key - diag + a.window_left;
  }
  Frag8 vf[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st)
    vf[st].v = key_ok && st * 16 + lh * 8 < Dr ? load16(vp + (size_t)my_key * k_rs + st * 16 + lh * 8)
                                               : u32x4{0, 0, 0, 0};  // zero past the head dimension
  f32x16 dkt[ND], dvt[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    dkt[d] = f32x16{};
    dvt[d] = f32x16{};
  }
  const int tr_row = 4 * lh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // Row reads (row li of a 32-row block, chunk 2 st + lh): offset li*D + ((2 st) ^ ry)*8.
  const int ry = lh ^ Swz::f(li);
  // Transposed reads of Q / dO: row 16 t + tr_row + 8 hi, column 32 d + tr_col of a tile.
  // With f = f(tr_row + 8 hi) the offset is trb[hi] + 32 (d ^ (f >> 2)) + 16 t D.
  int trb[2], trx[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const int r = tr_row + 8 * hi;
    const int f = Swz::f(r);
    trb[hi] = r * D + (tr_col & 7) + 8 * ((tr_col >> 3) ^ (f & 3));
    trx[hi] = f >> 2;
  }
  int ktr[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) ktr[hi] = Swz::elem(8 * lh + ((lane & 15) >> 2) + 4 * hi, (wave % ND) * 32 + tr_col);
  // this lane's 32 bytes in a stored dS tile: key row wave * 32 + li, positions 16 lh ..
  const int ds_lane = wave * 1024 + li * 32 + lh * 16;

  wait_all_memory();
  __syncthreads();

  auto step = [&](int it, int h, int i0, int h_next, int i0_next, bool mask, const uint16_t* __restrict__ Q,
                  const uint16_t* __restrict__ dO, const float* __restrict__ lse_c, const float* __restrict__ dsum_c,
                  uint16_t* __restrict__ Qn, uint16_t* __restrict__ dOn, float* __restrict__ lse_n,
                  float* __restrict__ dsum_n, uint16_t* __restrict__ dSc) {
    const float sl = sl_next;
    if (it + 1 < nsteps) fetch(h_next, i0_next, Qn, dOn, lse_n, dsum_n);

    bool live = true;  // some key of this wavefront is kept by some row of the step
    if constexpr (MASKED) {
      const int kw0 = k0 + wave * 32;
      live = !mask || (kw0 <= kw.hi(min(i0 + kK2BQ, Lq) - 1) && kw0 + 31 >= kw.lo(i0));
    }
    // dP starts from -Dsum of the step's rows (register r holds row 8 (r / 4) + 4 lh + r % 4),
    // so that the products leave dP - Dsum, and S from -LSE log2(e) / c, so that they leave
    // S - LSE / scale and P = exp2(c S) needs no LSE read after them.
    f32x16 s, dp;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 d4 = *(const f32x4*)(dsum_c + 8 * g4 + 4 * lh);
      const f32x4 l4 = *(const f32x4*)(lse_c + 8 * g4 + 4 * lh);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dp[4 * g4 + j] = d4[j];
        s[4 * g4 + j] = -l4[j] * inv_c;
      }
    }
    if (live) {
      // The row reads run SPD k-steps ahead of their products, written out in that order
      // and fenced for the machine scheduler (which would sink each read down to its
      // product and leave every product waiting for LDS).
      constexpr int SPD = 2;
      const int ryo = opaque(ry);
      Frag8 qa[SPD], ga[SPD], kf[SPD];
      auto issue = [&](auto st_tag) __attribute__((always_inline)) {
        constexpr int st = decltype(st_tag)::value, sl = st % SPD;
        const int ro = li * D + ((st * 2) ^ ryo) * 8;
        qa[sl].v = load16(Q + ro);
        ga[sl].v = load16(dO + ro);
        kf[sl].v = load16(Ks + wave * 32 * D + ro);
      };
      static_for<0, SPD>([&](auto st) __attribute__((always_inline)) { issue(st); });
      static_for<0, NS>([&](auto st_tag) __attribute__((always_inline)) {
        constexpr int st = decltype(st_tag)::value, sl = st % SPD;
        __builtin_amdgcn_sched_barrier(0);
        s = mfma32x32x16<BF16>(qa[sl], kf[sl], s);
        dp = mfma32x32x16<BF16>(ga[sl], vf[st], dp);
        if constexpr (st + SPD < NS) issue(Idx<st + SPD>{});
      });
      __builtin_amdgcn_sched_barrier(0);
    }
    if (__builtin_expect(mask, 0)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + 8 * (r >> 2) + 4 * lh + (r & 3);
        bool keep = live && key_ok && row < Lq;
        if constexpr (MASKED) keep = keep && row >= rmin && row <= rmax;
        s[r] = keep ? s[r] : -INFINITY;  // exp2(-inf) = 0: c is strictly positive
      }
    }
    // Register r holds query row i0 + 8 g4 + 4 lh + j (r = 4 g4 + j) of this lane's key.
    const float abase = (float)(i0 + 4 * lh + diag - my_key);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * g4 + j;
        float p;
        if constexpr (ALIBI) {
          p = fast_exp2(fmaf(s[r], c, -sl * fabsf(abase + (float)(8 * g4 + j))));
        } else {
          p = fast_exp2(s[r] * c);
        }
        s[r] = p;
        dp[r] = p * dp[r];  // dS / scale = P (dP - Dsum)
      }
    }
    Frag8 pf[2], dsf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r0 = 8 * t;
      pf[t].v = u32x4{pack2<BF16>(s[r0 + 0], s[r0 + 1]), pack2<BF16>(s[r0 + 2], s[r0 + 3]),
                      pack2<BF16>(s[r0 + 4], s[r0 + 5]), pack2<BF16>(s[r0 + 6], s[r0 + 7])};
      dsf[t].v = u32x4{pack2<BF16>(dp[r0 + 0], dp[r0 + 1]), pack2<BF16>(dp[r0 + 2], dp[r0 + 3]),
                       pack2<BF16>(dp[r0 + 4], dp[r0 + 5]), pack2<BF16>(dp[r0 + 6], dp[r0 + 7])};
    }
#pragma unroll
    for (int t = 0; t < (DQ ? 2 : 0); ++t) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t two = dsf[t].v[w];
        const int r = 8 * t + 2 * w;
        const int rl0 = 8 * (r >> 2) + 4 * lh + (r & 3);
        dSc[rl0 * SSTR + wave * 32 + li] = (uint16_t)(two & 0xffff);
        dSc[(rl0 + 1) * SSTR + wave * 32 + li] = (uint16_t)(two >> 16);
      }
    }
    if (live) {
      // dV^T += dO^T P^T and dK^T += Q^T dS^T over ops (t, d), transposed reads KPD ops
      // ahead in fenced order.
      constexpr int KPD = 2, NKO = 2 * ND;
      const int b0 = opaque(trb[0]), b1 = opaque(trb[1]);
      Frag8 ga[KPD], qa[KPD];
      auto issue = [&](auto op_tag) __attribute__((always_inline)) {
        constexpr int op = decltype(op_tag)::value, sl = op % KPD, t = op / ND, d = op % ND;
        const int o_lo = b0 + 32 * (d ^ trx[0]) + t * 16 * D;
        const int o_hi = b1 + 32 * (d ^ trx[1]) + t * 16 * D;
        const u32x2 g_lo = lds_read_tr16(dO + o_lo);
        const u32x2 g_hi = lds_read_tr16(dO + o_hi);
        const u32x2 q_lo = lds_read_tr16(Q + o_lo);
        const u32x2 q_hi = lds_read_tr16(Q + o_hi);
        ga[sl].v = u32x4{g_lo.x, g_lo.y, g_hi.x, g_hi.y};
        qa[sl].v = u32x4{q_lo.x, q_lo.y, q_hi.x, q_hi.y};
      };
      static_for<0, KPD>([&](auto op) __attribute__((always_inline)) { issue(op); });
      static_for<0, NKO>([&](auto op_tag) __attribute__((always_inline)) {
        constexpr int op = decltype(op_tag)::value, sl = op % KPD, t = op / ND, d = op % ND;
        __builtin_amdgcn_sched_barrier(0);
        dvt[d] = mfma32x32x16<BF16>(ga[sl], pf[t], dvt[d]);
        dkt[d] = mfma32x32x16<BF16>(qa[sl], dsf[t], dkt[d]);
        if constexpr (op + KPD < NKO) issue(Idx<op + KPD>{});
      });
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (DQ) {
      // This wavefront's prefetch of the next step has landed (and the dQ atomics it issued
      // before that prefetch have completed).  After the barrier every wavefront's dS is in
      // dSc, nobody reads this step's Q / dO / LSE / Dsum tiles any more, and the next
      // step's tiles are in LDS everywhere -- so no second barrier closes the step: the
      // wavefronts that compute this step's dQ overlap with the others starting the next
      // step, which writes its dS into the other buffer.
      wait_vmcnt<0>();
      lds_barrier();
      // dQ[32 rows][d-block] = dS[32 rows][256 keys] K[256 keys][d-block]: groups of ND
      // wavefronts take turns by step, one d-block per wavefront.
      if (wave / ND == it % (kK2Waves / ND)) {
        const int dblk = wave % ND;
        bool any = true;
        if (mask) any = i0 < Lq && k0 <= kw.hi(min(i0 + kK2BQ, Lq) - 1) && k_last >= kw.lo(i0);
        if (any) {
          f32x16 dq = f32x16{};
          // Operand reads QPD key steps ahead, in fenced order (as for S and dP above).
          constexpr int QPD = 3, NKS = kK2Keys / 16;
          Frag8 sa[QPD], kb2[QPD];
          auto issue = [&](auto ks_tag) __attribute__((always_inline)) {
            constexpr int ks = decltype(ks_tag)::value, sl = ks % QPD;
            sa[sl].v = load16(&dSc[li * SSTR + ks * 16 + lh * 8]);
            const u32x2 lo = lds_read_tr16(Ks + ks * 16 * D + ktr[0]);
            const u32x2 hi = lds_read_tr16(Ks + ks * 16 * D + ktr[1]);
            kb2[sl].v = u32x4{lo.x, lo.y, hi.x, hi.y};
          };
          static_for<0, QPD>([&](auto ks) __attribute__((always_inline)) { issue(ks); });
          static_for<0, NKS>([&](auto ks_tag) __attribute__((always_inline)) {
            constexpr int ks = decltype(ks_tag)::value, sl = ks % QPD;
            __builtin_amdgcn_sched_barrier(0);
            dq = mfma32x32x16<BF16>(sa[sl], kb2[sl], dq);
            if constexpr (ks + QPD < NKS) issue(Idx<ks + QPD>{});
          });
          __builtin_amdgcn_sched_barrier(0);
          // Buffer atomics from the step's first row: the row offset of register r is
          // uniform (scalar offset), the lane's row half and column form the lane offset.
          // The resource spans the rest of the accumulator, and rows past its B * Sq rows
          // (possible only with invalid cu_seqlens) are skipped: the scalar offset is not
          // range-checked by the hardware.
          const size_t acc0 = ((size_t)(q_start + i0) * a.Hq + h) * Dr;
          const auto dqr = make_rsrc(a.dq_acc + acc0, bytes_left(ws_rows * a.Hq * Dr, acc0, 4u));
          const uint32_t rs4 = (uint32_t)a.Hq * Dr * 4u;  // bytes per row
          const uint32_t voff = 4u * lh * rs4 + (uint32_t)(dblk * 32 + li) * 4u;
          // rows < lim are stored; columns past the head dimension are not (a d-block that
          // reaches past it takes the per-element path)
          const int lim = (int)min((size_t)Lq, ws_rows - min(ws_rows, (size_t)q_start));
          if (__builtin_expect(i0 + kK2BQ <= lim && (dblk + 1) * 32 <= Dr, 1)) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(dq[r], dqr, (int)voff, (int)((8 * (r >> 2) + (r & 3)) * rs4),
                                                            0);
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int rr = 8 * (r >> 2) + (r & 3);
              if (i0 + 4 * lh + rr < lim && dblk * 32 + li < Dr)
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(dq[r], dqr, (int)voff, (int)(rr * rs4), 0);
            }
          }
        }
      }
    } else {
      wait_vmcnt<0>();  // the prefetched step has landed
      lds_barrier();    // everywhere, and every wavefront is done with this step's tiles
      // Without dQ here, the route over stored dS keeps this wavefront's 32 keys x 32 rows
      // of dS / scale for the dQ pass: two 16-byte stores per lane, zeros where nothing is
      // kept (so every tile of the step range is written whole).  Issued after the wait, so
      // that they have a whole step to complete before the next one (the counter that
      // wait reads covers stores too).
      if (a.ds != nullptr && i0 / kK2BQ < a.ds_nqs) {  // (the step bound fails only for invalid cu_seqlens)
        uint16_t* t = a.ds + (((size_t)b * a.Hq + h) * a.ds_nqs + (size_t)(i0 / kK2BQ)) * a.ds_nkb * (kK2BQ * kK2Keys) +
                      (size_t)kb * (kK2BQ * kK2Keys);
        store16(t + ds_lane, dsf[0].v);
        store16(t + ds_lane + 8, dsf[1].v);
      }
    }
  };

  auto needs_mask = [&](int i0) {
    bool full = i0 + kK2BQ <= Lq && k0 + kK2Keys <= Lk;
    if constexpr (MASKED) full = full && kw.lo(i0 + kK2BQ - 1) <= k0 && kw.hi(i0) >= k0 + kK2Keys - 1;
    return !full;
  };
  int h_c = hk * G, q_c = qb_begin;  // this step's query head and block
  int h_n = h_c, q_n = q_c + 1;      // the next step's
  if (q_n == qb_end) {
    q_n = qb_begin;
    ++h_n;
  }
  for (int it = 0; it < nsteps; ++it) {
    const bool odd = it & 1;
    step(it, h_c, q_c * kK2BQ, h_n, q_n * kK2BQ, needs_mask(q_c * kK2BQ), odd ? Q1 : Q0, odd ? dO1 : dO0,
         odd ? lse1 : lse0, odd ? dsum1 : dsum0, odd ? Q0 : Q1, odd ? dO0 : dO1, odd ? lse0 : lse1,
         odd ? dsum0 : dsum1, odd ? dS1 : dS0);
    h_c = h_n;
    q_c = q_n;
    if (++q_n == qb_end) {
      q_n = qb_begin;
      ++h_n;
    }
  }

  if (key_ok) {
    uint16_t* dkp = (uint16_t*)a.dk + (size_t)(k_start + my_key) * k_rs + (size_t)hk * Dr;
    uint16_t* dvp = (uint16_t*)a.dv + (size_t)(k_start + my_key) * k_rs + (size_t)hk * Dr;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int col = d * 32 + 8 * gq + 4 * lh;
        u32x2 wk, wv;
        wk.x = pack2<BF16>(dkt[d][4 * gq + 0] * a.scale, dkt[d][4 * gq + 1] * a.scale);
        wk.y = pack2<BF16>(dkt[d][4 * gq + 2] * a.scale, dkt[d][4 * gq + 3] * a.scale);
        wv.x = pack2<BF16>(dvt[d][4 * gq + 0], dvt[d][4 * gq + 1]);
        wv.y = pack2<BF16>(dvt[d][4 * gq + 2], dvt[d][4 * gq + 3]);
        if (col < Dr) {  // four columns, all inside or all past the head dimension
          *(u32x2*)(dkp + col) = wk;
          *(u32x2*)(dvp + col) = wv;
        }
      }
    }
  }
}

// The key blocks of one launch, longest query range first (causal: ascending key block),
// are handed out from a queue in the workspace: a fixed grid of at most one workgroup per
// CU takes the next block whenever it finishes one.  Every CU stays busy until the queue
// runs dry, whatever the XCD and shader-engine placement of the workgroups and however the
// XCDs' speeds differ (the hardware dispatcher places workgroups in order, shader engine by
// shader engine, so a launch with one workgroup per block left CUs idle for tens of
// microseconds).  The preprocess empties the queue; the last workgroup to finish empties it
// again, so a main loop launched on its own (after a complete one) finds it empty too.
template <int D, bool BF16, bool MASKED, bool VARLEN, bool DQ, bool ALIBI>
__global__ __launch_bounds__(512, 1) void bwd_main_k256_kernel(BwdArgs a) {
  if (debug_stop(a.dbg)) return;
  __shared__ int next;
  const int nblocks = (a.Sk + kK2Keys - 1) / kK2Keys * a.B * a.Hkv;
  for (;;) {
    wait_all_memory();  // the previous block's loads into LDS and its atomics are done
    if (threadIdx.x == 0) next = (int)atomicAdd(a.work, 1u);
    __syncthreads();
    const int lin = next;
    __syncthreads();  // every wavefront has read it before it is overwritten
    if (lin >= nblocks) break;
    bwd_k256_block<D, BF16, MASKED, VARLEN, DQ, ALIBI>(a, lin);
  }
  if (threadIdx.x == 0 && atomicAdd(a.work + 1, 1u) == gridDim.x - 1) {
    // Every workgroup is past its last take from the queue.
    a.work[0] = 0;
    a.work[1] = 0;
  }
}

// ---------------------------------------------------------------- 2c. deterministic dQ pass

// dQ without atomics (the deterministic backward): one workgroup per (128-row query
// block, query head, sequence), walking its key tiles like the forward does, with P
// recomputed from the LSE instead of a running softmax:
//   S^T = K Q^T, dP^T = V dO^T, P = exp2(S c - LSE log2 e), dS = scale P (dP - Dsum),
//   dQ^T += K^T dS^T.
// Q and dO stay in registers as MFMA B operands; each lane holds one query row, so LSE
// and Dsum are per-lane scalars; K and V tiles stream through LDS double-buffered by
// direct loads; dQ accumulates in registers and is written once.  Every dQ element is
// the same sum in the same order on every run.
constexpr int kDqWaves = 4;
constexpr int kDqBM = 32 * kDqWaves;
constexpr int kDqBN = 64;

template <int D, bool BF16, bool MASKED, bool VARLEN, bool ALIBI>
__global__ __launch_bounds__(256, 2) void bwd_dq_pass_kernel(BwdArgs a) {
  if (debug_stop(a.dbg)) return;
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int TILE = kDqBN * D;
  using Swz = DualSwizzle<D>;
  __shared__ __attribute__((aligned(16))) uint16_t K0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t K1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int lh = lane >> 5;

  const int nqb = (a.Sq + kDqBM - 1) / kDqBM;
  const int nbh = a.B * a.Hq;
  const int qb = nqb - 1 - blockIdx.x / nbh;  // longest key loops first
  const int bh = blockIdx.x % nbh;
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;

  int q_start, k_start, Lq, Lk;
  if constexpr (VARLEN) {
    q_start = load_uniform(a.cu_q + b);
    Lq = load_uniform(a.cu_q + b + 1) - q_start;
    k_start = load_uniform(a.cu_k + b);
    Lk = load_uniform(a.cu_k + b + 1) - k_start;
  } else {
    q_start = b * a.Sq;
    Lq = a.Sq;
    k_start = b * a.Sk;
    Lk = a.Sk;
  }
  const int q0 = qb * kDqBM;
  if (q0 >= Lq) return;  // uniform

  const int hk = h / (a.Hq / a.Hkv);
  const int Dr = a.D;  // head dimension of the tensors (<= D, the tile width)
  const int Dc = Dr / 8;
  const size_t q_rs = (size_t)a.Hq * Dr;
  const size_t k_rs = (size_t)a.Hkv * Dr;
  const uint16_t* qp = (const uint16_t*)a.q + (size_t)q_start * q_rs + (size_t)h * Dr;
  const uint16_t* dop = (const uint16_t*)a.dout + (size_t)q_start * q_rs + (size_t)h * Dr;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)k_start * k_rs + (size_t)hk * Dr;
  const uint16_t* vp = (const uint16_t*)a.v + (size_t)k_start * k_rs + (size_t)hk * Dr;

  const int diag = Lk - Lq;
  KeyWindow kw{Lk, diag, 0, -1, -1};
  if constexpr (MASKED) kw = KeyWindow{Lk, diag, a.causal, a.window_left, a.window_right};
  const int last_row = min(q0 + kDqBM, Lq) - 1;
  const int k_lo = kw.lo(q0), k_hi = kw.hi(last_row);
  const int kb_begin = k_lo / kDqBN;
  const int kb_end = k_hi >= k_lo ? k_hi / kDqBN + 1 : kb_begin;
  const int all_lo = kw.lo(last_row), all_hi = kw.hi(q0);
  const int my_row = q0 + wave * 32 + li;
  const bool row_ok = my_row < Lq;
  const int wave_row0 = q0 + wave * 32;
  const int wave_lo = kw.lo(wave_row0), wave_hi = kw.hi(min(wave_row0 + 31, Lq - 1));
  const int my_lo = kw.lo(my_row), my_hi = kw.hi(my_row);

  constexpr int NI = TILE / 8 / 256;
  uint32_t foff[NI];  // bytes
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int chunk = (i * kDqWaves + wave) * 64 + lane;
    const int r = chunk / Swz::CH;
    foff[i] = (uint32_t)(r * (int)k_rs + src_chunk(Swz::chunk(r, chunk % Swz::CH), Dc) * 8) * 2u;
  }
  // Buffer-form direct loads from the tile's first key (the flat form would make the
  // compiler wait for every LDS read of the loop with lgkmcnt(0)).
  const size_t k_rows = VARLEN ? (size_t)load_uniform(a.cu_k + a.B) : (size_t)a.B * a.Sk;
  auto fetch = [&](int kb, uint16_t* __restrict__ Kd, uint16_t* __restrict__ Vd) {
    const int k0 = kb * kDqBN;
    const size_t kfirst = (size_t)(k_start + k0) * k_rs + (size_t)hk * Dr;
    const uint32_t kbytes = bytes_left(k_rows * k_rs, kfirst, 2u);
    const auto kr = make_rsrc((const uint16_t*)a.k + kfirst, kbytes);
    const auto vr = make_rsrc((const uint16_t*)a.v + kfirst, kbytes);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int first = (i * kDqWaves + wave) * 64;
      uint32_t off = foff[i];
      if (k0 + kDqBN > Lk) {
        const int chunk = first + lane;
        const int r = chunk / Swz::CH;
        off = (uint32_t)(min(r, Lk - 1 - k0) * (int)k_rs + src_chunk(Swz::chunk(r, chunk % Swz::CH), Dc) * 8) * 2u;
      }
      lds_buffer_load16(kr, off, Kd + first * 8);
      lds_buffer_load16(vr, off, Vd + first * 8);
    }
  };
  if (kb_begin < kb_end) fetch(kb_begin, K0, V0);

  Frag8 qf[NS], gf[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    // zero past the head dimension (the padded K / V chunks re-read chunk 0)
    const bool in = row_ok && st * 16 + lh * 8 < Dr;
    qf[st].v = in ? load16(qp + (size_t)my_row * q_rs + st * 16 + lh * 8) : u32x4{0, 0, 0, 0};
    gf[st].v = in ? load16(dop + (size_t)my_row * q_rs + st * 16 + lh * 8) : u32x4{0, 0, 0, 0};
  }
  constexpr float kLog2e = 1.4426950408889634f;
  float lse2 = INFINITY, dsum = 0.f;
  if (row_ok) {
    size_t li_idx;
    if constexpr (VARLEN) {
      li_idx = (size_t)h * load_uniform(a.cu_q + a.B) + q_start + my_row;
    } else {
      li_idx = ((size_t)b * a.Hq + h) * a.Sq + my_row;
    }
    lse2 = a.lse[li_idx] * kLog2e;
    dsum = a.dsum[(size_t)(q_start + my_row) * a.Hq + h];
  }
  const float c = a.scale_log2;
  float sl2 = 0.f;  // ALiBi slope in exp2 units
  if constexpr (ALIBI) sl2 = a.alibi[(size_t)b * a.alibi_bstride + h] * kLog2e;
  const int row_diag = my_row + diag;

  f32x16 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = f32x16{};
  const int tr_row = 4 * lh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int ry = lh ^ Swz::f(li);  // row reads: li*D + ((2 st) ^ ry)*8
  int trb[2], trx[2];               // transposed reads: trb[hi] + 32 (d ^ trx[hi]) + 16 t D
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const int r = tr_row + 8 * hi;
    const int f = Swz::f(r);
    trb[hi] = r * D + (tr_col & 7) + 8 * ((tr_col >> 3) ^ (f & 3));
    trx[hi] = f >> 2;
  }

  wait_all_memory();
  __syncthreads();

  auto tile = [&](int kb, bool mask, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                  uint16_t* __restrict__ Kn, uint16_t* __restrict__ Vn) {
    const int k0 = kb * kDqBN;
    if (kb + 1 < kb_end) fetch(kb + 1, Kn, Vn);
    if (!(mask && (k0 > wave_hi || k0 + kDqBN - 1 < wave_lo))) {  // some key of the tile is kept
      f32x16 s[2], dp[2];
      const int ryo = opaque(ry);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        s[sub] = f32x16{};
        dp[sub] = f32x16{};
      }
      {
        // S^T and dP^T: op o = (sub, st), its K and V row reads issued RA ops ahead in
        // fenced order (left to itself the scheduler sinks each read down to its product).
        constexpr int RA = 2, NO = 2 * NS;
        Frag8 kf[RA], vf[RA];
        auto issue = [&](auto o_tag) __attribute__((always_inline)) {
          constexpr int o = decltype(o_tag)::value, sl = o % RA, sub = o / NS, st = o % NS;
          const int ro = (sub * 32 + li) * D + ((st * 2) ^ ryo) * 8;
          kf[sl].v = load16(K + ro);
          vf[sl].v = load16(V + ro);
        };
        static_for<0, RA>([&](auto o) __attribute__((always_inline)) { issue(o); });
        static_for<0, NO>([&](auto o_tag) __attribute__((always_inline)) {
          constexpr int o = decltype(o_tag)::value, sl = o % RA, sub = o / NS, st = o % NS;
          __builtin_amdgcn_sched_barrier(0);
          s[sub] = mfma32x32x16<BF16>(kf[sl], qf[st], s[sub]);
          dp[sub] = mfma32x32x16<BF16>(vf[sl], gf[st], dp[sub]);
          if constexpr (o + RA < NO) issue(Idx<o + RA>{});
        });
        __builtin_amdgcn_sched_barrier(0);
      }
      if (__builtin_expect(mask, 0)) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + sub * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            s[sub][r] = (key >= my_lo && key <= my_hi) ? s[sub][r] : -INFINITY;
          }
      }
      Frag8 df[4];
      const float abase = (float)(k0 + 4 * lh - row_diag);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float bias = -lse2;
          if constexpr (ALIBI) bias = fmaf(-sl2, fabsf(abase + (float)(sub * 32 + 8 * (r >> 2) + (r & 3))), bias);
          const float p = fast_exp2(fmaf(s[sub][r], c, bias));
          s[sub][r] = a.scale * p * (dp[sub][r] + dsum);  // the workspace holds -Dsum
        }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int sub = t >> 1, r0 = (t & 1) * 8;
        df[t].v = u32x4{pack2<BF16>(s[sub][r0 + 0], s[sub][r0 + 1]), pack2<BF16>(s[sub][r0 + 2], s[sub][r0 + 3]),
                        pack2<BF16>(s[sub][r0 + 4], s[sub][r0 + 5]), pack2<BF16>(s[sub][r0 + 6], s[sub][r0 + 7])};
      }
      const int b0 = opaque(trb[0]), b1 = opaque(trb[1]);
      {
        // dQ^T += K^T dS^T: op o = (t, d), transposed K reads RA ops ahead, fenced.
        constexpr int RA = 2, NO = 4 * ND;
        Frag8 kt[RA];
        auto issue = [&](auto o_tag) __attribute__((always_inline)) {
          constexpr int o = decltype(o_tag)::value, sl = o % RA, t = o / ND, d = o % ND;
          const u32x2 lo = lds_read_tr16(K + b0 + 32 * (d ^ trx[0]) + t * 16 * D);
          const u32x2 hi = lds_read_tr16(K + b1 + 32 * (d ^ trx[1]) + t * 16 * D);
          kt[sl].v = u32x4{lo.x, lo.y, hi.x, hi.y};
        };
        static_for<0, RA>([&](auto o) __attribute__((always_inline)) { issue(o); });
        static_for<0, NO>([&](auto o_tag) __attribute__((always_inline)) {
          constexpr int o = decltype(o_tag)::value, sl = o % RA, t = o / ND, d = o % ND;
          __builtin_amdgcn_sched_barrier(0);
          acc[d] = mfma32x32x16<BF16>(kt[sl], df[t], acc[d]);
          if constexpr (o + RA < NO) issue(Idx<o + RA>{});
        });
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_all_memory();
    __syncthreads();
  };

  for (int kb = kb_begin; kb < kb_end; ++kb) {
    const bool odd = (kb - kb_begin) & 1;
    const int k0 = kb * kDqBN;
    const bool full = k0 >= all_lo && k0 + kDqBN - 1 <= all_hi;
    tile(kb, !full, odd ? K1 : K0, odd ? V1 : V0, odd ? K0 : K1, odd ? V0 : V1);
  }

  if (row_ok) {
    uint16_t* gp = (uint16_t*)a.dq + (size_t)(q_start + my_row) * q_rs + (size_t)h * Dr;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = d * 32 + 8 * g + 4 * lh;
        u32x2 w;
        w.x = pack2<BF16>(acc[d][4 * g + 0], acc[d][4 * g + 1]);
        w.y = pack2<BF16>(acc[d][4 * g + 2], acc[d][4 * g + 3]);
        if (col < Dr) *(u32x2*)(gp + col) = w;
      }
    }
  }
}

// ---------------------------------------------------------------- 2d. dQ from stored dS

// dQ = scale dS K from the dS tiles the main loop stored (the route with neither dQ
// atomics nor a second computation of S and dP): one workgroup per (128-row query block,
// query head, sequence), four wavefronts of one 32-row query step each, two workgroups per
// CU.  The key blocks of the main loop that reach the workgroup's steps are walked in
// stages of 64 keys (32 at D = 256) through a double-buffered LDS ring filled by direct
// loads: the stage's K rows, shared, and each wavefront's slice of its own dS tile.  (The
// ring takes up to four slots; deeper rings measured slower: the compiler then waits for
// the direct loads of the previous stage before every LDS read, as it cannot tell the
// slots apart across stages.)  dQ^T += K^T dS^T accumulates on MFMA with both operands taken by
// transposed LDS reads (K^T from the swizzled K rows; dS^T from the stored key rows, whose
// 64 bytes hold the 32 query rows in the order the main loop's products produced them).
// A wavefront skips the key blocks whose step range does not hold its step (those tiles
// were never written).  dQ is written once: the same sum in the same order on every run.
// Every stored dS element is read once; the pass is bound by those reads.

// Wavefronts (32-row query steps) per workgroup, and keys per LDS stage (two stages,
// double-buffered, so that two workgroups fit on a CU and one streams while the other
// multiplies).
constexpr int ds_waves(int) { return 4; }
constexpr int ds_stage_keys(int D) { return D == 256 ? 32 : 64; }

// LDS ring slot i of a stage ring held as distinct objects (so that the compiler can tell
// the reads of one slot from the direct loads in flight into another).
template <int I, class T>
__device__ __forceinline__ T* ring_slot(T* s0, T* s1, T* s2, T* s3) {
  if constexpr (I == 0) return s0;
  else if constexpr (I == 1) return s1;
  else if constexpr (I == 2) return s2;
  else return s3;
}

template <int D, bool BF16>
__global__ __launch_bounds__(64 * ds_waves(D), 2) void bwd_dq_ds_kernel(BwdArgs a) {
  if (debug_stop(a.dbg)) return;
  constexpr int kDsWaves = ds_waves(D);
  constexpr int kDsRows = 32 * kDsWaves;  // query rows per workgroup
  constexpr int kDsSK = ds_stage_keys(D);
  constexpr int KB = bwd_block_keys(D);  // keys per main-loop block (one stored tile)
  constexpr int TILE = 32 * KB;          // elements of a stored tile
  constexpr int SPB = KB / kDsSK;        // stages per key block
  constexpr int NST = 2;                 // ring depth (LDS: 64 KiB at D = 128, 48 KiB at 64 and 256)
  constexpr int ND = D / 32;
  constexpr int KT = kDsSK * D;          // K elements per stage
  constexpr int STW = kDsSK * 32;        // dS elements per wavefront per stage (key rows of 32)
  constexpr int NK = KT / 8 / (64 * kDsWaves);  // 16-byte K loads per lane per stage
  constexpr int NSL = STW / 8 / 64;      // 16-byte dS loads per lane per stage
  constexpr int L = NK + NSL;            // vector-memory loads per lane per stage, in every wavefront
  static_assert(KB % kDsSK == 0 && kDsSK % 16 == 0 && NK >= 1 && NSL >= 1 && (NST - 2) * L < 64, "stage shape");
  using Swz = DualSwizzle<D>;
  __shared__ __attribute__((aligned(16))) uint16_t K0[KT];
  __shared__ __attribute__((aligned(16))) uint16_t K1[KT];
  __shared__ __attribute__((aligned(16))) uint16_t K2[NST > 2 ? KT : 8];
  __shared__ __attribute__((aligned(16))) uint16_t K3[NST > 3 ? KT : 8];
  __shared__ __attribute__((aligned(16))) uint16_t S0[kDsWaves * STW];
  __shared__ __attribute__((aligned(16))) uint16_t S1[kDsWaves * STW];
  __shared__ __attribute__((aligned(16))) uint16_t S2[NST > 2 ? kDsWaves * STW : 8];
  __shared__ __attribute__((aligned(16))) uint16_t S3[NST > 3 ? kDsWaves * STW : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int lh = lane >> 5;

  const int nqb = (a.Sq + kDsRows - 1) / kDsRows;
  const int nbh = a.B * a.Hq;
  const int qb = nqb - 1 - (int)blockIdx.x / nbh;  // causal: the longest key ranges first
  const int bh = (int)blockIdx.x % nbh;
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;

  const bool varlen = a.cu_q != nullptr;
  int q_start, k_start, Lq, Lk;
  if (varlen) {
    q_start = load_uniform(a.cu_q + b);
    Lq = load_uniform(a.cu_q + b + 1) - q_start;
    k_start = load_uniform(a.cu_k + b);
    Lk = load_uniform(a.cu_k + b + 1) - k_start;
  } else {
    q_start = b * a.Sq;
    Lq = a.Sq;
    k_start = b * a.Sk;
    Lk = a.Sk;
  }
  if (qb * kDsRows >= Lq) return;  // uniform

  const bool masked = a.causal || a.window_left >= 0 || a.window_right >= 0;
  const int hk = h / (a.Hq / a.Hkv);
  const int Dr = a.D;  // head dimension of the tensors (<= D, the tile width)
  const int Dc = Dr / 8;
  const size_t q_rs = (size_t)a.Hq * Dr;
  const size_t k_rs = (size_t)a.Hkv * Dr;
  const int step0 = qb * kDsWaves;               // the workgroup's first query step
  const int my_step = step0 + wave;               // this wavefront's
  const int nsteps_seq = (Lq + 31) / 32;
  const int last_step = min(step0 + kDsWaves, nsteps_seq) - 1;
  const int nkb = Lk > 0 ? (Lk + KB - 1) / KB : 0;

  // Key blocks whose step range reaches one of the workgroup's steps: [kb_lo, kb_hi].
  // (The ranges move forward with the key block, so these are contiguous.)
  int kb_lo = nkb, kb_hi = -1;
  for (int kb = 0; kb < nkb; ++kb) {
    const StepRange r = block_steps(kb * KB, KB, Lq, Lk, masked, a.causal, a.window_left, a.window_right);
    if (r.begin <= last_step && r.end > step0) {
      kb_lo = min(kb_lo, kb);
      kb_hi = kb;
    }
  }
  const int nst = kb_hi >= kb_lo ? (kb_hi - kb_lo + 1) * SPB : 0;

  // Direct loads of stage s: its 64 K rows (clamped to the sequence; the padding chunks
  // past the head dimension re-read chunk 0 and only feed dQ columns that are never
  // stored) into the shared K slot, and this wavefront's 64 key rows of its dS tile into its
  // part of the dS slot.  A wavefront whose step the block does not reach still loads (from
  // its step clamped into the array, never used), so that every wavefront issues L loads per
  // stage and the waits below can count them.
  const size_t k_rows = varlen ? (size_t)load_uniform(a.cu_k + a.B) : (size_t)a.B * a.Sk;
  const uint16_t* ds_head = a.ds + ((size_t)b * a.Hq + h) * a.ds_nqs * a.ds_nkb * (size_t)TILE;
  const size_t my_tiles = (size_t)min(my_step, a.ds_nqs - 1) * a.ds_nkb * (size_t)TILE;
  auto issue = [&](int s, uint16_t* __restrict__ Kd, uint16_t* __restrict__ Sd) {
    const int kb = kb_lo + s / SPB;
    const int kbase = kb * KB;  // < Lk
    const int k0 = kbase + (s % SPB) * kDsSK;
    const size_t kfirst = (size_t)(k_start + kbase) * k_rs + (size_t)hk * Dr;
    const auto kr = make_rsrc((const uint16_t*)a.k + kfirst, min(bytes_left(k_rows * k_rs, kfirst, 2u), 0x7fffffffu));
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int first = (i * kDsWaves + wave) * 64;
      const int chunk = first + lane;
      const int r = chunk / Swz::CH;
      const int g = Swz::chunk(r, chunk % Swz::CH);
      const int key = min(k0 + r, Lk - 1) - kbase;  // 0 <= key < KB
      lds_buffer_load16(kr, (uint32_t)(key * (int)k_rs + src_chunk(g, Dc) * 8) * 2u, Kd + first * 8);
    }
    // (the clamps of step and key block to the area bind only for invalid cu_seqlens)
    const auto sr = make_rsrc(ds_head + my_tiles + (size_t)min(kb, a.ds_nkb - 1) * TILE + (s % SPB) * STW, STW * 2u);
#pragma unroll
    for (int i = 0; i < NSL; ++i)
      lds_buffer_load16_stream(sr, (uint32_t)(i * 64 + lane) * 16u, Sd + wave * STW + i * 512);
  };

  // Transposed-read bases.  K^T (A operand): lane reads key rows 8 lh + (lane & 15) / 4 + 4 hi
  // of a 16-key step, columns 32 d + tr_col (swizzled: k_base[hi] + 32 (d ^ k_x[hi]));
  // dS^T (B operand): key rows as for K, positions 16 ((lane >> 4) & 1) + 4 (lane & 3).
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int k_base[2], k_x[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const int r = 8 * lh + ((lane & 15) >> 2) + 4 * hi;
    const int f = Swz::f(r);
    k_base[hi] = r * D + 8 * ((tr_col >> 3) ^ (f & 3)) + (tr_col & 7);
    k_x[hi] = f >> 2;
  }
  const int s_base = wave * STW + (8 * lh + ((lane & 15) >> 2)) * 32 + tr_col;

  f32x16 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = f32x16{};

  auto compute = [&](const uint16_t* __restrict__ K, const uint16_t* __restrict__ S) {
    // ops o = (16-key step ks, d-block d); operand reads RA ops ahead in fenced order.
    constexpr int NO = (kDsSK / 16) * ND, RA = 2;
    const int kb0 = opaque(k_base[0]), kb1 = opaque(k_base[1]);
    Frag8 kt[RA], sf[2];
    auto read = [&](auto o_tag) __attribute__((always_inline)) {
      constexpr int o = decltype(o_tag)::value, sl = o % RA, ks = o / ND, d = o % ND;
      const u32x2 lo = lds_read_tr16(K + ks * 16 * D + kb0 + 32 * (d ^ k_x[0]));
      const u32x2 hi = lds_read_tr16(K + ks * 16 * D + kb1 + 32 * (d ^ k_x[1]));
      kt[sl].v = u32x4{lo.x, lo.y, hi.x, hi.y};
      if constexpr (d == 0) {
        const u32x2 slo = lds_read_tr16(S + s_base + ks * 16 * 32);
        const u32x2 shi = lds_read_tr16(S + s_base + ks * 16 * 32 + 4 * 32);
        sf[ks & 1].v = u32x4{slo.x, slo.y, shi.x, shi.y};
      }
    };
    static_for<0, RA>([&](auto o) __attribute__((always_inline)) { read(o); });
    static_for<0, NO>([&](auto o_tag) __attribute__((always_inline)) {
      constexpr int o = decltype(o_tag)::value, sl = o % RA, ks = o / ND, d = o % ND;
      __builtin_amdgcn_sched_barrier(0);
      acc[d] = mfma32x32x16<BF16>(kt[sl], sf[ks & 1], acc[d]);
      if constexpr (o + RA < NO) read(Idx<o + RA>{});
    });
    __builtin_amdgcn_sched_barrier(0);
  };

  // The whole ring walk in one function that takes the slots as distinct restrict
  // pointers, so that the compiler can tell the reads of a stage from the direct loads in
  // flight into the other slots (issued in this or an earlier stage) and does not wait for
  // those before every read.  Stage s: wait for its loads, barrier, issue the loads of
  // stage s + NST - 1 into the slot stage s - 1 used, then this wavefront's products.
  auto walk = [&](uint16_t* __restrict__ k0, uint16_t* __restrict__ k1, uint16_t* __restrict__ k2,
                  uint16_t* __restrict__ k3, uint16_t* __restrict__ s0p, uint16_t* __restrict__ s1p,
                  uint16_t* __restrict__ s2p, uint16_t* __restrict__ s3p) __attribute__((always_inline)) {
    static_for<0, NST - 1>([&](auto j_tag) __attribute__((always_inline)) {
      constexpr int j = decltype(j_tag)::value;
      if (j < nst) issue(j, ring_slot<j>(k0, k1, k2, k3), ring_slot<j>(s0p, s1p, s2p, s3p));
    });
    for (int s0 = 0; s0 < nst; s0 += NST) {
      static_for<0, NST>([&](auto j_tag) __attribute__((always_inline)) {
        constexpr int j = decltype(j_tag)::value;
        const int s = s0 + j;
        if (s < nst) {
          // Stage s has landed once at most the loads of the stages issued after it are in
          // flight (loads complete in issue order; nothing else is outstanding here).
          if (s + NST - 2 < nst) {
            wait_vmcnt<(NST - 2) * L>();
          } else {
            wait_vmcnt<0>();
          }
          // Every wavefront's loads of stage s are in LDS, and every wavefront is done with
          // stage s - 1, whose slot the next issue reuses.
          lds_barrier();
          if (s + NST - 1 < nst)
            issue(s + NST - 1, ring_slot<(j + NST - 1) % NST>(k0, k1, k2, k3),
                  ring_slot<(j + NST - 1) % NST>(s0p, s1p, s2p, s3p));
          const int kb = kb_lo + s / SPB;
          const StepRange r = block_steps(kb * KB, KB, Lq, Lk, masked, a.causal, a.window_left, a.window_right);
          if (r.begin <= my_step && my_step < r.end) compute(ring_slot<j>(k0, k1, k2, k3), ring_slot<j>(s0p, s1p, s2p, s3p));
        }
      });
    }
  };
  walk(K0, K1, K2, K3, S0, S1, S2, S3);

  // Lane li holds query row position li of the step (row = the position's bits permuted as
  // in the stored tile) and, in register r of d-block d, column 32 d + 8 (r / 4) + 4 lh + r % 4.
  const int row = my_step * 32 + 16 * ((li >> 3) & 1) + 8 * ((li >> 2) & 1) + 4 * (li >> 4) + (li & 3);
  const size_t q_rows = varlen ? (size_t)load_uniform(a.cu_q + a.B) : (size_t)a.B * a.Sq;
  if (row < Lq && (size_t)(q_start + row) < q_rows) {
    uint16_t* gp = (uint16_t*)a.dq + (size_t)(q_start + row) * q_rs + (size_t)h * Dr;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = d * 32 + 8 * g + 4 * lh;
        u32x2 w;
        w.x = pack2<BF16>(acc[d][4 * g + 0] * a.scale, acc[d][4 * g + 1] * a.scale);
        w.y = pack2<BF16>(acc[d][4 * g + 2] * a.scale, acc[d][4 * g + 3] * a.scale);
        if (col < Dr) *(u32x2*)(gp + col) = w;
      }
    }
  }
}

// ---------------------------------------------------------------- 3. finalize

template <bool BF16, bool VARLEN>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  if (debug_stop(a.dbg)) return;
  // 8 elements per thread
  size_t rows = (size_t)a.B * a.Sq;  // the workspace's rows (a bound on total_q)
  if constexpr (VARLEN) rows = min(rows, (size_t)max(load_uniform(a.cu_q + a.B), 0));
  const size_t n8 = rows * a.Hq * a.D / 8;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
    const u32x4 x0 = load16(a.dq_acc + i * 8);
    const u32x4 x1 = load16(a.dq_acc + i * 8 + 4);
    const float* f0 = (const float*)&x0;
    const float* f1 = (const float*)&x1;
    u32x4 o;
    const float sc = a.scale;  // the main loops accumulate dS K with dS / scale
    o.x = pack2<BF16>(f0[0] * sc, f0[1] * sc);
    o.y = pack2<BF16>(f0[2] * sc, f0[3] * sc);
    o.z = pack2<BF16>(f1[0] * sc, f1[1] * sc);
    o.w = pack2<BF16>(f1[2] * sc, f1[3] * sc);
    store16((uint16_t*)a.dq + i * 8, o);
  }
}

// ---------------------------------------------------------------- launch

// Compute units of the current device (the backward main loop runs one workgroup per CU).
int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  return n;
}

template <int D, bool BF16, bool MASKED, bool VARLEN, bool ALIBI>
hipError_t launch_bwd_t(const BwdArgs& a, int stages, hipStream_t stream) {
  const size_t rows = (size_t)a.B * a.Sq;  // bound on total_q in varlen mode
  if (stages & kBwdPre) {
    constexpr int PAIRS = 256 / (D / 8);
    const size_t pairs = rows * a.Hq;
    const dim3 grid((unsigned)((pairs + PAIRS - 1) / PAIRS));
    hipLaunchKernelGGL((bwd_pre_kernel<D, BF16, VARLEN>), grid, dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & (kBwdMainAtomic | kBwdRecompute | kBwdMainStoreDs)) {
    // the main loop without dQ serves the recompute route and, with a.ds set, the
    // stored-dS route
    const bool det = (stages & kBwdMainAtomic) == 0;
    if constexpr (D <= 128) {
      const int nkb = (a.Sk + kK2Keys - 1) / kK2Keys;
      const dim3 grid((unsigned)std::min(nkb * a.B * a.Hkv, cu_count()));
      if (det) {
        hipLaunchKernelGGL((bwd_main_k256_kernel<D, BF16, MASKED, VARLEN, false, ALIBI>), grid, dim3(512), 0, stream, a);
      } else {
        hipLaunchKernelGGL((bwd_main_k256_kernel<D, BF16, MASKED, VARLEN, true, ALIBI>), grid, dim3(512), 0, stream, a);
      }
    } else {
      const int nkb = (a.Sk + kBwdBN - 1) / kBwdBN;
      const dim3 grid((unsigned)nkb * a.B * a.Hkv);
      if (det) {
        hipLaunchKernelGGL((bwd_main_kernel<D, BF16, MASKED, VARLEN, false, ALIBI>), grid, dim3(256), 0, stream, a);
      } else {
        hipLaunchKernelGGL((bwd_main_kernel<D, BF16, MASKED, VARLEN, true, ALIBI>), grid, dim3(256), 0, stream, a);
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (stages & kBwdRecompute) {
      const int nqb = (a.Sq + kDqBM - 1) / kDqBM;
      const dim3 grid((unsigned)nqb * a.B * a.Hq);
      hipLaunchKernelGGL((bwd_dq_pass_kernel<D, BF16, MASKED, VARLEN, ALIBI>), grid, dim3(256), 0, stream, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (stages & kBwdDqFromDs) {
    constexpr int rows = 32 * ds_waves(D);
    const int nqb = (a.Sq + rows - 1) / rows;
    hipLaunchKernelGGL((bwd_dq_ds_kernel<D, BF16>), dim3((unsigned)nqb * a.B * a.Hq), dim3(64 * ds_waves(D)), 0, stream,
                       a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kBwdFinalize) {
    const size_t n8 = rows * a.Hq * a.D / 8;
    size_t blocks = (n8 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL((bwd_dq_kernel<BF16, VARLEN>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D, bool BF16, bool MASKED>
hipError_t launch_bwd_m(const BwdArgs& a, int st, hipStream_t stream) {
  const bool varlen = a.cu_q != nullptr;
  if (a.alibi != nullptr) {
    return varlen ? launch_bwd_t<D, BF16, MASKED, true, true>(a, st, stream)
                  : launch_bwd_t<D, BF16, MASKED, false, true>(a, st, stream);
  }
  return varlen ? launch_bwd_t<D, BF16, MASKED, true, false>(a, st, stream)
                : launch_bwd_t<D, BF16, MASKED, false, false>(a, st, stream);
}

template <int D, bool BF16>
hipError_t launch_bwd_d(const BwdArgs& a, int st, hipStream_t stream) {
  const bool masked = a.causal || a.window_left >= 0 || a.window_right >= 0;
  return masked ? launch_bwd_m<D, BF16, true>(a, st, stream) : launch_bwd_m<D, BF16, false>(a, st, stream);
}

template <int D>
hipError_t launch_bwd_dt(const BwdArgs& a, int st, hipStream_t stream) {
  return a.bf16 ? launch_bwd_d<D, true>(a, st, stream) : launch_bwd_d<D, false>(a, st, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int stage_mask, hipStream_t stream) {
  switch (tile_headdim(a.D)) {
    case 64: return launch_bwd_dt<64>(a, stage_mask, stream);
    case 128: return launch_bwd_dt<128>(a, stage_mask, stream);
    case 256: return launch_bwd_dt<256>(a, stage_mask, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
