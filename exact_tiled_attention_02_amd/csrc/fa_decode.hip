// Decode against a read-only KV cache: a few query rows per sequence, a long cache, the
// keys split over many workgroups ("split-KV"), then a separate merge of the partials.
//
// Method (FlashAttention README, changelog entry 2.2 "optimise for inference" and the
// flash_attn_with_kvcache docstring): with very short queries the cost is reading the KV
// cache, so the keys of one sequence are divided among workgroups that each produce a
// partial output and its log-sum-exp, and a second kernel combines them.  The merge is
// exact in real arithmetic: LSE = ln sum_r exp(LSE_r), O = sum_r exp(LSE_r - LSE) O_r.
// Cache addressing follows the same docstring: per-sequence lengths (cache_seqlens), an
// optional indirection to the cache entry (cache_batch_idx), or a paged cache addressed
// through a block table; the causal mask and the sliding window are aligned to the
// bottom-right corner with seqlen_k = cache_seqlens[b]; ALiBi adds
// -slope * |i + seqlen_k - seqlen_q - j| to the scaled score.
//
// Work layout (MI355X):
//   * the query rows of the G = Hq / Hkv query heads that read one KV head are processed
//     together -- row r = s * G + g for query s and head g of the group -- so every byte
//     of the cache is read once per KV head; 32 rows form the N side of one MFMA tile
//     (S^T = K Q^T, one query row per lane as in the prefill forward);
//   * one wavefront per workgroup, owning a contiguous range of key tiles of one
//     (sequence, KV head, row group).  Tiles of 32 keys go from global memory straight
//     into a ring of STAGES LDS slots private to the wavefront (global_load_lds_dwordx4),
//     STAGES - 1 tiles ahead of the one being multiplied; a tile is ready when the
//     wavefront's own vmcnt says so, so no workgroup barrier is needed.  The kernel is
//     HBM-bound, so what matters is the bytes in flight per CU: rings of 48 KiB (three
//     workgroups per CU, 96 KiB in flight) measured best for D = 64 and 128;
//   * masking runs only on tiles at the edges of the kept range;
//   * the block table of a paged cache is read once into a register per lane (page p of
//     the split in lane p) and picked per tile with v_readlane, so no memory access sits
//     between two tile loads.
#include <mutex>
#include <type_traits>

#include "fa.h"
#include "fa_device.h"
#include "fa_params.h"

namespace fa {
namespace {

constexpr int kDecKeys = 32;  // keys per tile
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.4426950408889634f;


// Keys [lo, hi] kept for query s of a sequence with Lk keys and Sq queries.
struct KeyRange {
  int lo, hi;
};
__device__ __forceinline__ KeyRange kept_keys(int s, int Lk, int Sq, int causal, int wl, int wr) {
  const int diag = s + Lk - Sq;
  KeyRange k;
  k.lo = wl >= 0 ? max(0, diag - wl) : 0;
  k.hi = Lk - 1;
  if (causal) k.hi = min(k.hi, diag);
  if (wr >= 0) k.hi = min(k.hi, diag + wr);
  return k;
}

template <int D, bool BF16, bool PAGED, bool ALIBI>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
  if (debug_stop(a.dbg)) return;
  constexpr int STAGES = decode_stages(D);
  constexpr int NS = D / 16;            // 16-wide slices of the head dimension
  constexpr int ND = D / 32;            // 32-wide output blocks
  constexpr int TILE = kDecKeys * D;    // elements of one K (or V) tile
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int NI = TILE / 8 / 64;     // direct loads per tensor per tile
  constexpr int LPT = 2 * NI;           // vector-memory operations per tile
  static_assert((STAGES - 1) * LPT < 64, "vmcnt holds 6 bits");
  using Swz = DualSwizzle<D>;
  // One LDS object per ring slot (K tile then V tile), always addressed statically: the
  // compiler then knows that reading one slot does not touch the loads in flight into
  // the others and does not wait for them.  Slots beyond STAGES are never referenced
  // and take no LDS.
  __shared__ __attribute__((aligned(16))) uint16_t S0[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t S1[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t S2[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t S3[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t S4[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t S5[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t S6[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t S7[2 * TILE];
  auto slot = [&](auto k) __attribute__((always_inline)) -> uint16_t* {
    constexpr int K = decltype(k)::value;
    static_assert(K < STAGES, "slot");
    if constexpr (K == 0) return S0;
    else if constexpr (K == 1) return S1;
    else if constexpr (K == 2) return S2;
    else if constexpr (K == 3) return S3;
    else if constexpr (K == 4) return S4;
    else if constexpr (K == 5) return S5;
    else if constexpr (K == 6) return S6;
    else return S7;
  };

  const int lane = threadIdx.x;
  const int li = lane & 31;
  const int lh = lane >> 5;

  // Block -> work item.  Blocks are dealt to the 8 XCDs round-robin (block x runs on XCD
  // x % 8).  A group is one (sequence, KV head, split); groups are ordered split-major
  // (split 0 of every sequence and KV head first) with the KV head fastest, so at any
  // time the running groups cover many sequences and all heads and the later, shorter
  // splits fill the tail; the row groups of one group follow each other on one XCD and
  // share its L2.  (Measured on MI355X against other orders: contiguous ranges per XCD
  // and split-fastest orders were 5-30% slower on ragged caches.)
  const int n_groups = a.B * a.Hkv * a.splits;
  const int xcd = (int)(blockIdx.x & 7);
  const int j = (int)(blockIdx.x >> 3);
  const int group = (j / a.row_groups) * 8 + xcd;
  const int rg = j % a.row_groups;
  if (group >= n_groups) return;
  const int hk = group % a.Hkv;
  const int b = (group / a.Hkv) % a.B;
  const int split = group / a.Hkv / a.B;

  const int G = a.Hq / a.Hkv;
  const int M = a.Sq * G;
  int Lk = a.cap;
  if (a.cache_seqlens != nullptr) Lk = min(max(a.cache_seqlens[b], 0), a.cap);

  // This lane's query row.
  const int r = rg * 32 + li;
  const bool row_ok = r < M;
  const int s = row_ok ? r / G : 0;
  const int h = hk * G + (row_ok ? r % G : 0);
  const int diag = s + Lk - a.Sq;
  KeyRange mine = kept_keys(s, Lk, a.Sq, a.causal, a.window_left, a.window_right);
  if (!row_ok) mine = KeyRange{0, 0x3fffffff};

  // Key range of the row group (the ranges grow with s) and the part every row keeps.
  const int s_first = rg * 32 / G;
  const int s_last = min(M - 1, rg * 32 + 31) / G;
  const KeyRange first = kept_keys(s_first, Lk, a.Sq, a.causal, a.window_left, a.window_right);
  const KeyRange last = kept_keys(s_last, Lk, a.Sq, a.causal, a.window_left, a.window_right);
  const int lo_all = last.lo, hi_all = first.hi;
  int t_begin = 0, t_end = 0;
  if (Lk > 0 && last.hi >= first.lo) {
    t_begin = first.lo / kDecKeys;
    t_end = last.hi / kDecKeys + 1;
  }
  // Splits are chunks of a fixed number of tiles (set by the host from the capacity, so
  // that every split of every sequence costs at most the same); a split past the end of
  // a shorter sequence is empty and only writes its empty partial.
  const int t0 = min(t_end, t_begin + split * a.chunk_tiles);
  const int t1 = min(t_end, t0 + a.chunk_tiles);

  const int Dr = a.D;  // head dimension of the tensors (<= D, the tile width)
  const int Dc = Dr / 8;
  const size_t rs = (size_t)a.Hkv * Dr;  // elements between consecutive keys
  const uint16_t* kbase = (const uint16_t*)a.k + (size_t)hk * Dr;
  const uint16_t* vbase = (const uint16_t*)a.v + (size_t)hk * Dr;
  int bt = 0, pfirst = 0, ipg = 0, ioff = 0;
  if constexpr (PAGED) {
    pfirst = t0 * kDecKeys / a.page;
    ipg = pfirst;
    ioff = t0 * kDecKeys - pfirst * a.page;
    const int p = pfirst + lane;
    if (t0 < t1 && p < a.max_blocks) bt = a.block_table[(size_t)b * a.max_blocks + p];
  } else {
    const int entry = a.cache_batch_idx != nullptr ? a.cache_batch_idx[b] : b;
    kbase += (size_t)entry * a.entry_stride;
    vbase += (size_t)entry * a.entry_stride;
  }

  // Per-lane source offsets of the direct loads within a tile (LDS chunk c of row rr
  // receives the global chunk c ^ f(rr)).
  uint32_t foff[NI];  // bytes
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int chunk = i * 64 + lane;
    const int rr = chunk / CH;
    foff[i] = (uint32_t)(rr * (int)rs + src_chunk(Swz::chunk(rr, chunk % CH), Dc) * 8) * 2u;
  }

  // Issue the loads of tile t into ring slot k.  Tiles are issued in increasing order,
  // which advances the page cursor (ipg, ioff) of a paged cache.
  auto issue = [&](int t, auto k) __attribute__((always_inline)) {
    uint16_t* dst = slot(k);
    const int k0 = t * kDecKeys;
    const uint16_t* kt;
    const uint16_t* vt;
    if constexpr (PAGED) {
      const int phys = __builtin_amdgcn_readlane(bt, ipg - pfirst);
      const size_t row0 = (size_t)phys * a.page + ioff;
      kt = kbase + row0 * rs;
      vt = vbase + row0 * rs;
      ioff += kDecKeys;
      if (ioff == a.page) {
        ioff = 0;
        ++ipg;
      }
    } else {
      kt = kbase + (size_t)k0 * rs;
      vt = vbase + (size_t)k0 * rs;
    }
    if (k0 + kDecKeys <= Lk) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        lds_direct_load16(kt, foff[i], dst + i * 512);
        lds_direct_load16(vt, foff[i], dst + TILE + i * 512);
      }
    } else {
      // Rows past the last key re-read the last key (finite data, masked to P = 0); they
      // stay inside the tile's page.
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int chunk = i * 64 + lane;
        const int rr = chunk / CH;
        const uint32_t off =
            (uint32_t)(min(rr, Lk - 1 - k0) * (int)rs + src_chunk(Swz::chunk(rr, chunk % CH), Dc) * 8) * 2u;
        lds_direct_load16(kt, off, dst + i * 512);
        lds_direct_load16(vt, off, dst + TILE + i * 512);
      }
    }
  };

  // Q^T operand (B of S^T = K Q^T): lane holds Q[row][16 st + 8 lh .. +7].
  const uint16_t* qp = (const uint16_t*)a.q + ((size_t)(b * a.Sq + s) * a.Hq + h) * Dr;
  Frag8 qf[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st)  // zero past the head dimension (padded K chunks re-read chunk 0)
    qf[st].v = row_ok && st * 16 + lh * 8 < Dr ? load16(qp + st * 16 + lh * 8) : u32x4{0, 0, 0, 0};
  float sl2 = 0.f;  // ALiBi slope in exp2 units
  if constexpr (ALIBI) sl2 = row_ok ? a.alibi[(size_t)b * a.alibi_bstride + h] * kLog2e : 0.f;

  // The page list (and everything above) must have arrived before the first tile load is
  // counted by vmcnt.
  wait_all_memory();

  static_for<0, STAGES - 1>([&](auto k) __attribute__((always_inline)) {
    if (t0 + decltype(k)::value < t1) issue(t0 + decltype(k)::value, k);
  });

  f32x16 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = f32x16{};
  float m_run = -INFINITY;  // running max of the exp2-domain scores
  float l_run = 0.f;
  const float c = a.scale_log2;

  const int tr_row = 4 * lh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int koff[NS], voff[2][ND];
#pragma unroll
  for (int st = 0; st < NS; ++st) koff[st] = Swz::row_elem(li, st * 2 + lh);
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int d = 0; d < ND; ++d) voff[hi][d] = Swz::elem(tr_row + 8 * hi, d * 32 + tr_col);

  auto compute = [&](int t, auto k) __attribute__((always_inline)) {
    const uint16_t* Kt = slot(k);
    const uint16_t* Vt = Kt + TILE;
    const int k0 = t * kDecKeys;
    f32x16 sc = f32x16{};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      Frag8 kf;
      kf.v = load16(Kt + koff[st]);
      sc = mfma32x32x16<BF16>(kf, qf[st], sc);
    }
    // Register r holds key k0 + 8 (r / 4) + 4 lh + r % 4 of this lane's row.
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = sc[e] * c;
      if constexpr (ALIBI) {
        const int key = k0 + 8 * (e >> 2) + 4 * lh + (e & 3);
        x = fmaf(-sl2, fabsf((float)(diag - key)), x);
      }
      sc[e] = x;
    }
    if (__builtin_expect(k0 < lo_all || k0 + kDecKeys - 1 > hi_all, 0)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 8 * (e >> 2) + 4 * lh + (e & 3);
        sc[e] = (key >= mine.lo && key <= mine.hi) ? sc[e] : -INFINITY;
      }
    }
    float mx = m_run;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[e]);
    mx = pair_max(mx);
    const float m_use = mx == -INFINITY ? 0.f : mx;
    const float alpha = fast_exp2(m_run - m_use);  // 0 while nothing was kept
    m_run = mx;
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = fast_exp2(sc[e] - m_use);
      sc[e] = p;
      ls += p;
    }
    l_run = l_run * alpha + ls;
    if (__builtin_expect(__any(alpha != 1.f), 0)) {
#pragma unroll
      for (int d = 0; d < ND; ++d) acc[d] *= alpha;
    }
    // P^T slices of 16 keys as B operands; V^T from transposed LDS reads.
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
      Frag8 pf;
      const int e0 = ts * 8;
      pf.v = u32x4{pack2<BF16>(sc[e0 + 0], sc[e0 + 1]), pack2<BF16>(sc[e0 + 2], sc[e0 + 3]),
                   pack2<BF16>(sc[e0 + 4], sc[e0 + 5]), pack2<BF16>(sc[e0 + 6], sc[e0 + 7])};
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const u32x2 lo = lds_read_tr16(Vt + ts * 16 * D + voff[0][d]);
        const u32x2 hi = lds_read_tr16(Vt + ts * 16 * D + voff[1][d]);
        Frag8 vf;
        vf.v = u32x4{lo.x, lo.y, hi.x, hi.y};
        acc[d] = mfma32x32x16<BF16>(vf, pf, acc[d]);
      }
    }
  };

  // Tile t sits in slot (t - t0) % STAGES.  Before multiplying it, issue tile
  // t + STAGES - 1 into the slot freed by tile t - 1, then wait until tile t has landed:
  // at most (tiles issued after it) * LPT loads may still be outstanding.
  auto step = [&](int t, auto k) __attribute__((always_inline)) {
    constexpr int K = decltype(k)::value;
    if (t + STAGES - 1 < t1) issue(t + STAGES - 1, std::integral_constant<int, (K + STAGES - 1) % STAGES>{});
    const int after = min(STAGES - 1, t1 - 1 - t);
    static_for<0, STAGES>([&](auto n) __attribute__((always_inline)) {
      if (after == decltype(n)::value) wait_vmcnt<decltype(n)::value * LPT>();
    });
    compute(t, k);
  };
  int t = t0;
  for (; t + STAGES <= t1; t += STAGES) {
    static_for<0, STAGES>([&](auto k) __attribute__((always_inline)) { step(t + decltype(k)::value, k); });
  }
  static_for<0, STAGES - 1>([&](auto k) __attribute__((always_inline)) {
    if (t + decltype(k)::value < t1) step(t + decltype(k)::value, k);
  });

  // Epilogue: this lane's row, columns 32 d + 8 g + 4 lh .. +3 of block d.
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_nat = m_run * kLn2 + __logf(l_tot);
  const size_t orow = (size_t)(b * a.Sq + s) * a.Hq + h;
  const size_t lrow = ((size_t)b * a.Hq + h) * a.Sq + s;
  if (!row_ok) return;
  if (a.splits == 1) {
    uint16_t* op = (uint16_t*)a.out + orow * Dr;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w.x = pack2<BF16>(acc[d][4 * g + 0] * inv, acc[d][4 * g + 1] * inv);
        w.y = pack2<BF16>(acc[d][4 * g + 2] * inv, acc[d][4 * g + 3] * inv);
        if (d * 32 + 8 * g + 4 * lh < Dr) *(u32x2*)(op + d * 32 + 8 * g + 4 * lh) = w;
      }
    }
    if (lh == 0) a.lse[lrow] = l_tot > 0.f ? lse_nat : INFINITY;
  } else {
    const size_t nrows = (size_t)a.B * a.Sq * a.Hq;
    float* op = a.o_part + ((size_t)split * nrows + orow) * Dr;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w = {acc[d][4 * g + 0] * inv, acc[d][4 * g + 1] * inv, acc[d][4 * g + 2] * inv,
                   acc[d][4 * g + 3] * inv};
        if (d * 32 + 8 * g + 4 * lh < Dr) *(f32x4*)(op + d * 32 + 8 * g + 4 * lh) = w;
      }
    }
    if (lh == 0) a.lse_part[(size_t)split * nrows + lrow] = l_tot > 0.f ? lse_nat : -INFINITY;
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Merge of the split partials: one wavefront per output row (b, s, h).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  if (debug_stop(a.dbg)) return;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nrows = a.B * a.Sq * a.Hq;
  const int row = blockIdx.x * 4 + wave;
  if (row >= nrows) return;
  const int h = row % a.Hq;
  const int bs = row / a.Hq;
  const int s = bs % a.Sq;
  const int b = bs / a.Sq;
  const size_t lrow = ((size_t)b * a.Hq + h) * a.Sq + s;
  const int S = a.splits;
  const float* lp = a.lse_part + lrow;

  float mx = -INFINITY;
  for (int r = lane; r < S; r += 64) mx = fmaxf(mx, lp[(size_t)r * nrows]);
  mx = wave_max(mx);
  const int Dr = a.D;  // head dimension (<= D)
  uint16_t* op = (uint16_t*)a.out + (size_t)row * Dr;
  if (mx == -INFINITY) {  // no split kept a key: zero output, LSE +inf
    for (int e = lane; e < Dr; e += 64) op[e] = 0;
    if (lane == 0) a.lse[lrow] = INFINITY;
    return;
  }
  float sum = 0.f;
  for (int r = lane; r < S; r += 64) sum += __expf(lp[(size_t)r * nrows] - mx);
  const float L = mx + __logf(wave_sum(sum));

  // Lanes cover (split, 4-column chunk) pairs; partials of an empty split are zeros with
  // weight exp(-inf) = 0.
  constexpr int C4 = D / 4;
  constexpr int RPI = 64 / C4;  // splits per pass
  const int c4 = lane % C4;
  const int rsub = lane / C4;
  const bool col_ok = c4 * 4 < Dr;  // lanes past the head dimension add zeros and store nothing
  const float* pp = a.o_part + (size_t)row * Dr + c4 * 4;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int r = rsub; r < S; r += RPI) {
    const float w = __expf(lp[(size_t)r * nrows] - L);
    const f32x4 x = col_ok ? *(const f32x4*)(pp + (size_t)r * nrows * Dr) : f32x4{0.f, 0.f, 0.f, 0.f};
    o += w * x;
  }
#pragma unroll
  for (int off = C4; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] += __shfl_xor(o[e], off);
  }
  if (rsub == 0 && col_ok) {
    u32x2 w;
    w.x = pack2<BF16>(o[0], o[1]);
    w.y = pack2<BF16>(o[2], o[3]);
    *(u32x2*)(op + c4 * 4) = w;
  }
  if (lane == 0) a.lse[lrow] = L;
}

template <int D, bool BF16, bool PAGED, bool ALIBI>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const long long groups = (long long)a.B * a.Hkv * a.splits;
  const long long blocks = (groups + 7) / 8 * 8 * a.row_groups;
  hipLaunchKernelGGL((decode_kernel<D, BF16, PAGED, ALIBI>), dim3((unsigned)blocks), dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const int nrows = a.B * a.Sq * a.Hq;
  hipLaunchKernelGGL((decode_combine_kernel<D, BF16>), dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  const bool paged = a.block_table != nullptr;
  const bool alibi = a.alibi != nullptr;
  if (paged) {
    return alibi ? launch_decode_t<D, BF16, true, true>(a, stream) : launch_decode_t<D, BF16, true, false>(a, stream);
  }
  return alibi ? launch_decode_t<D, BF16, false, true>(a, stream) : launch_decode_t<D, BF16, false, false>(a, stream);
}

template <int D>
hipError_t launch_decode_dt(const DecodeArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_decode_d<D, true>(a, stream) : launch_decode_d<D, false>(a, stream);
}

}  // namespace

namespace {

// Partial results of fa_fwd_kvcache_noalloc, for callers that cannot allocate: a static
// array of the library, one copy on each device it runs on, held until the process ends.
// Host code must not use this name as an address (on the host it is only a stand-in for
// the symbol): the device address comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) unsigned char scratch[FA_KVCACHE_NOALLOC_MAX_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device ordinal

}  // namespace

hipError_t kvcache_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));  // with device `dev` current
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  switch (tile_headdim(a.D)) {
    case 64: return launch_decode_dt<64>(a, stream);
    case 128: return launch_decode_dt<128>(a, stream);
    case 256: return launch_decode_dt<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
