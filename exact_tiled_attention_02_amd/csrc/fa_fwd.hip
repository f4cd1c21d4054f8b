// Forward kernel: exact attention, one workgroup per (query block, query head, sequence).
//
// Method (FlashAttention README, "How to use FlashAttention"; FlashAttention-2 abstract
// as quoted on the flash-attention-2 snippet page; softmax details from the release
// notes "v1.4 - FlashAttention Fork", section 4):
//   * work is split over sequences, heads and 128-row query blocks; inside a workgroup
//     each of the 4 wavefronts owns 32 query rows, so the softmax statistics of a row
//     never leave its wavefront;
//   * the query tile stays in registers; key/value tiles of 64 rows stream through LDS,
//     double-buffered: the tile after the current one is fetched straight from global
//     memory into LDS (global_load_lds_dwordx4, no register staging) while the current
//     one is being multiplied, with one workgroup barrier per tile;
//   * per key tile: S^T = K Q^T on MFMA (fp32 accumulate), masking only on tiles that
//     touch the causal diagonal or the sequence tail, a running row max m and row sum l,
//     P = exp2(S * scale*log2(e) - m * scale*log2(e)) (one FMA + exp2), rescaling of the
//     output accumulator by exp2((m_old - m_new) * scale*log2(e)) on every tile (exact:
//     only a multiplication by exactly 1.0f is left out), then O^T += V^T P^T on MFMA
//     with P rounded once to 16 bits;
//   * a row max of -inf (nothing kept yet) is replaced by 0 so that no (-inf) - (-inf)
//     appears;
//   * epilogue: O = acc / l, LSE = m * scale + ln l; a row that kept no key writes O = 0
//     and LSE = +inf.
// Masks (flash_attn_func docstring: causal and window paragraphs, alibi_slopes): query i
// keeps keys lo(i) <= j <= hi(i) with the causal limit and the sliding window aligned to
// the bottom-right corner (KeyWindow).  A workgroup visits only the key tiles its rows can
// see; tiles inside every row's range carry no masking code, the rest set masked scores
// to -inf.  ALiBi adds -slope * |i + Lk - Lq - j| to the scaled score; that variant runs
// the softmax on exp2-domain scores t = S * scale*log2(e) + bias*log2(e) directly.
//
// Orientation: computing S^T (keys x query rows) puts one query row in each lane (and
// its twin lane l^32), so row reductions are in-lane plus one cross-half exchange
// (v_permlane32_swap), the per-row rescale is a per-lane scalar, and the fp32
// accumulator, converted to 16 bits, is already the B operand of the P V product.  V^T,
// the A operand of that product, is read from the row-major V tile with
// ds_read_b64_tr_b16.
//
// LDS tiles are unpadded and XOR-swizzled on 16-byte chunks (see DualSwizzle), which is
// what a direct global->LDS load can produce and keeps both read patterns free of bank
// conflicts.
#include <type_traits>

#include "fa_device.h"
#include "fa_params.h"

namespace fa {
namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdBM = 32 * kFwdWaves;  // query rows per workgroup
constexpr int kFwdBN = 64;              // keys per tile

// Workgroup -> (sequence b, query head h, query block qb); false: no work.
//
// Workgroups are dealt to the eight XCDs in turn (workgroup w runs on XCD w % 8, in the
// order of w within its XCD), and every XCD has an L2 of its own.  When Hq is a multiple
// of 8, XCD x takes the query heads [x Hq/8, (x+1) Hq/8) of every sequence: an equal
// share of the work, with the query heads of a KV head kept together.  Within the XCD:
//   * few blocks (at most four per CU): query blocks longest first over all of the XCD's
//     (sequence, head) pairs, which balances the CUs best;
//   * otherwise sequence by sequence, longest sequence first, the query blocks of a
//     sequence longest first with the heads of a block adjacent.  The workgroups resident
//     on the XCD at one time then stream the K/V tiles of one or two sequences, which its
//     L2 fetches once for all of them (packed batches of short sequences gain ~25 %).
// Otherwise (and for more than 64 packed sequences): query blocks longest first over all
// (sequence, head) pairs of the grid.  Blocks past a packed sequence's end report no work.
constexpr int kQbMajorMaxBlocks = 4 * 32;  // per XCD: four rounds of its 32 CUs

template <int BM, bool VARLEN>
__device__ __forceinline__ bool fwd_block(const FwdArgs& a, int& b, int& h, int& qb) {
  const int lin = blockIdx.x;
  const int nqb = (a.Sq + BM - 1) / BM;
  if ((a.Hq & 7) == 0 && (!VARLEN || a.B <= 64)) {
    const int x = lin & 7, t = lin >> 3;
    const int hx = a.Hq >> 3;
    // Lane i: the length of packed sequence i and its block count on this XCD.
    const int lane = threadIdx.x & 63;
    int len = 0, cnt = 0, total = nqb * hx * a.B;
    if constexpr (VARLEN) {
      len = lane < a.B ? a.cu_q[lane + 1] - a.cu_q[lane] : 0;
      cnt = (len + BM - 1) / BM * hx;
      total = cnt;
      for (int o = 32; o >= 1; o >>= 1) total += __shfl_xor(total, o);
      total = __builtin_amdgcn_readfirstlane(total);  // equal in every lane
    }
    if (total <= kQbMajorMaxBlocks) {
      const int per = a.B * hx;
      qb = nqb - 1 - t / per;
      b = (t % per) / hx;
      h = x * hx + t % hx;
      return true;
    }
    int cnt_b, pre_b;  // this XCD's blocks of the chosen sequence, and of those before it
    if constexpr (VARLEN) {
      // Rank by length (ties by index): count the blocks of the sequences ranked before.
      int pre = 0;
      for (int j = 0; j < a.B; ++j) {
        const int lj = __builtin_amdgcn_readlane(len, j);
        const int cj = __builtin_amdgcn_readlane(cnt, j);
        pre += (lj > len || (lj == len && j < lane)) ? cj : 0;
      }
      const uint64_t mine = __ballot(lane < a.B && t >= pre && t < pre + cnt);
      if (mine == 0) return false;
      b = (int)__builtin_ctzll(mine);
      cnt_b = __builtin_amdgcn_readlane(cnt, b);
      pre_b = __builtin_amdgcn_readlane(pre, b);
    } else {
      cnt_b = nqb * hx;
      b = t / cnt_b;
      pre_b = b * cnt_b;
    }
    const int u = t - pre_b;
    qb = cnt_b / hx - 1 - u / hx;
    h = x * hx + u % hx;
    b = __builtin_amdgcn_readfirstlane(b);  // uniform: keeps what is built from it scalar
    return true;
  }
  const int nbh = a.B * a.Hq;
  qb = nqb - 1 - lin / nbh;
  h = (lin % nbh) % a.Hq;
  b = (lin % nbh) / a.Hq;
  return true;
}

template <int D, bool BF16, bool MASKED, bool VARLEN, bool ALIBI>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  if (debug_stop(a.dbg)) return;
  constexpr int NS = D / 16;  // 16-wide slices of the head dimension (QK^T depth)
  constexpr int ND = D / 32;  // 32-wide blocks of the head dimension (output tiles)
  constexpr int TILE = kFwdBN * D;  // elements per K or V tile
  using Swz = DualSwizzle<D>;
  // Two buffers per tensor as distinct LDS objects, always addressed statically: the
  // compiler can then tell that reads of one buffer do not touch the direct loads in
  // flight into the other, and lets them overlap.
  __shared__ __attribute__((aligned(16))) uint16_t K0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t K1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS bases
  const int li = lane & 31;
  const int lh = lane >> 5;

  // Workgroup -> (query block, head, sequence).  Query blocks are visited from the last
  // one down, so under a causal mask the longest key loops start first.
  int b, h, qb;
  if (!fwd_block<kFwdBM, VARLEN>(a, b, h, qb)) return;  // uniform over the workgroup

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
  const int q0 = qb * kFwdBM;
  if (q0 >= Lq) return;  // uniform over the workgroup

  const int hk = h / (a.Hq / a.Hkv);
  const int Dr = a.D;  // head dimension of the tensors (<= D, the tile width)
  const int Dc = Dr / 8;
  const size_t q_rs = (size_t)a.Hq * Dr;
  const size_t k_rs = (size_t)a.Hkv * Dr;
  const uint16_t* qp = (const uint16_t*)a.q + (size_t)q_start * q_rs + (size_t)h * Dr;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)k_start * k_rs + (size_t)hk * Dr;
  const uint16_t* vp = (const uint16_t*)a.v + (size_t)k_start * k_rs + (size_t)hk * Dr;

  // Kept keys of row i: [kw.lo(i), kw.hi(i)], both non-decreasing in i.  Without a mask
  // every row keeps [0, Lk - 1].
  const int diag = Lk - Lq;
  KeyWindow kw{Lk, diag, 0, -1, -1};
  if constexpr (MASKED) kw = KeyWindow{Lk, diag, a.causal, a.window_left, a.window_right};
  const int last_row = min(q0 + kFwdBM, Lq) - 1;
  // Tiles any row of the block can see, and the key range that every row keeps.
  const int k_lo = kw.lo(q0), k_hi = kw.hi(last_row);
  const int kb_begin = k_lo / kFwdBN;
  const int kb_end = k_hi >= k_lo ? k_hi / kFwdBN + 1 : kb_begin;
  const int all_lo = kw.lo(last_row), all_hi = kw.hi(q0);

  const int my_row = q0 + wave * 32 + li;
  const bool row_ok = my_row < Lq;
  const int wave_row0 = q0 + wave * 32;
  const int wave_lo = kw.lo(wave_row0), wave_hi = kw.hi(min(wave_row0 + 31, Lq - 1));
  const int my_lo = kw.lo(my_row), my_hi = kw.hi(my_row);

  // Direct global->LDS fetch of key/value tile kb into buffer buf.  The per-lane source
  // offsets do not depend on the tile; only a tile reaching past the end of the
  // sequence needs its rows clamped (they re-read the last row: finite data, masked to
  // P = 0).
  constexpr int NI = TILE / 8 / 256;  // direct loads per wavefront per tensor
  uint32_t foff[NI];  // bytes
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int chunk = (i * kFwdWaves + wave) * 64 + lane;
    const int r = chunk / Swz::CH;
    foff[i] = (uint32_t)(r * (int)k_rs + src_chunk(Swz::chunk(r, chunk % Swz::CH), Dc) * 8) * 2u;
  }
  auto fetch = [&](int kb, auto buf_tag) {
    uint16_t* Kd = decltype(buf_tag)::value ? K1 : K0;
    uint16_t* Vd = decltype(buf_tag)::value ? V1 : V0;
    const int k0 = kb * kFwdBN;
    const uint16_t* kt = kp + (size_t)k0 * k_rs;
    const uint16_t* vt = vp + (size_t)k0 * k_rs;
    if (k0 + kFwdBN <= Lk) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int first = (i * kFwdWaves + wave) * 64;
        lds_direct_load16(kt, foff[i], Kd + first * 8);
        lds_direct_load16(vt, foff[i], Vd + first * 8);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int first = (i * kFwdWaves + wave) * 64;
        const int chunk = first + lane;
        const int r = chunk / Swz::CH;
        const uint32_t off =
            (uint32_t)(min(r, Lk - 1 - k0) * (int)k_rs + src_chunk(Swz::chunk(r, chunk % Swz::CH), Dc) * 8) * 2u;
        lds_direct_load16(kt, off, Kd + first * 8);
        lds_direct_load16(vt, off, Vd + first * 8);
      }
    }
  };

  // Processing order: first the run of tiles inside the key range every row keeps (an
  // even number of them, without masking code), then the remaining edge tiles -- those
  // before the run (window) and after it (diagonal, tail) -- with masking.  The online
  // softmax does not depend on the order.  Tiles alternate between the two buffers in
  // processing order, so both loops advance in pairs and name the buffers statically.
  const int u0 = min(max(kb_begin, (all_lo + kFwdBN - 1) / kFwdBN), kb_end);
  int u1 = all_hi >= 0 ? min(kb_end, (all_hi + 1) / kFwdBN) : 0;
  u1 = u1 > u0 ? u0 + ((u1 - u0) & ~1) : u0;
  const int n_lead = u0 - kb_begin;
  const int n_mask = n_lead + (kb_end - u1);
  auto masked_kb = [&](int j) { return j < n_lead ? kb_begin + j : u1 + (j - n_lead); };
  if (u1 > u0) {
    fetch(u0, std::false_type{});
  } else if (n_mask > 0) {
    fetch(masked_kb(0), std::false_type{});
  }

  // Q^T operand: lane holds Q[my_row][16 s + 8 lh .. +7] for every slice s.
  Frag8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    // zero past the head dimension: the padded K chunks re-read chunk 0 (src_chunk)
    qf[s].v = row_ok && s * 16 + lh * 8 < Dr ? load16(qp + (size_t)my_row * q_rs + s * 16 + lh * 8)
                                             : u32x4{0, 0, 0, 0};
  }

  f32x16 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = f32x16{};
  float m_run = -INFINITY;  // running max: raw scores, or exp2-domain scores with ALiBi
  float l_run = 0.f;
  const float c = a.scale_log2;
  constexpr float kLog2e = 1.4426950408889634f;
  float sl2 = 0.f;  // ALiBi slope in exp2 units, and this row's diagonal key
  if constexpr (ALIBI) sl2 = a.alibi[(size_t)b * a.alibi_bstride + h] * kLog2e;
  const int row_diag = my_row + diag;

  const int tr_row = 4 * lh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // Per-lane LDS offsets of the operand reads, fixed for the whole loop: row reads of K
  // (key row li, chunk 2 st + lh) and transposed reads of V (rows tr_row and tr_row + 8
  // of each 16-key slice, columns d*32 + tr_col); a slice or sub-block only adds a
  // constant.
  int koff[NS], voff[2][ND];
#pragma unroll
  for (int st = 0; st < NS; ++st) koff[st] = Swz::row_elem(li, st * 2 + lh);
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int d = 0; d < ND; ++d) voff[hi][d] = Swz::elem(tr_row + 8 * hi, d * 32 + tr_col);

  wait_all_memory();
  __syncthreads();

  // One key tile.  MASK selects the variant for tiles at the edges of the kept range
  // (causal diagonal, window borders, sequence tail); interior tiles carry no masking
  // code at all.
  auto tile = [&](int kb, int next, auto mask_tag, auto buf_tag) {
    constexpr bool BUF = decltype(buf_tag)::value;
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = kb * kFwdBN;
    if (next >= 0) fetch(next, std::integral_constant<bool, !BUF>{});

    // A wavefront whose rows keep no key of this tile has nothing to add.
    if (!(MASK && (k0 > wave_hi || k0 + kFwdBN - 1 < wave_lo))) {
      const uint16_t* K = BUF ? K1 : K0;
      const uint16_t* V = BUF ? V1 : V0;
      // S^T (keys x rows): two 32-key blocks.
      f32x16 s[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        s[sub] = f32x16{};
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          Frag8 kf;
          kf.v = load16(K + sub * 32 * D + koff[st]);
          s[sub] = mfma32x32x16<BF16>(kf, qf[st], s[sub]);
        }
      }

      // ALiBi: scores move to the exp2 domain with the bias added,
      // t = S c - slope log2(e) |key - (row + diag)|.
      if constexpr (ALIBI) {
        const float base = (float)(k0 + 4 * lh - row_diag);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float dist = base + (float)(sub * 32 + 8 * (r >> 2) + (r & 3));
            s[sub][r] = fmaf(-sl2, fabsf(dist), s[sub][r] * c);
          }
      }
      // Masked scores become -inf, so their probabilities are exp2(-inf) = 0 (the factor c
      // is strictly positive).  Only tiles at the edges of the kept range need it.
      if constexpr (MASK) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + sub * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            s[sub][r] = (key >= my_lo && key <= my_hi) ? s[sub][r] : -INFINITY;
          }
        }
      }

      float mx = m_run;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
      mx = pair_max(mx);
      const float m_use = (mx == -INFINITY) ? 0.f : mx;
      float alpha;
      float ls = 0.f;
      if constexpr (ALIBI) {
        alpha = fast_exp2(m_run - m_use);  // 0 while nothing was kept
        m_run = mx;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(s[sub][r] - m_use);
            s[sub][r] = p;
            ls += p;
          }
      } else {
        alpha = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_use) * c);
        m_run = mx;
        const float mc = m_use * c;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(s[sub][r], c, -mc));
            s[sub][r] = p;
            ls += p;
          }
      }
      l_run = l_run * alpha + ls;
      // Rescale the accumulator; when no row of the wavefront changed its maximum every
      // factor is exactly 1.0f and the multiplication is skipped (bitwise identical).
      if (__builtin_expect(__any(alpha != 1.f), 0)) {
#pragma unroll
        for (int d = 0; d < ND; ++d) acc[d] *= alpha;
      }

      // P^T as the B operand of O^T += V^T P^T: slice t covers keys 16t .. 16t+15; lane
      // position p of half lh stands for key 16t + 8(p/4) + 4lh + p%4.
      Frag8 pf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int sub = t >> 1, r0 = (t & 1) * 8;
        pf[t].v = u32x4{pack2<BF16>(s[sub][r0 + 0], s[sub][r0 + 1]), pack2<BF16>(s[sub][r0 + 2], s[sub][r0 + 3]),
                        pack2<BF16>(s[sub][r0 + 4], s[sub][r0 + 5]), pack2<BF16>(s[sub][r0 + 6], s[sub][r0 + 7])};
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const u32x2 lo = lds_read_tr16(V + t * 16 * D + voff[0][d]);
          const u32x2 hi = lds_read_tr16(V + t * 16 * D + voff[1][d]);
          Frag8 vf;
          vf.v = u32x4{lo.x, lo.y, hi.x, hi.y};
          acc[d] = mfma32x32x16<BF16>(vf, pf[t], acc[d]);
        }
      }
    }
    wait_all_memory();  // the prefetched tile has landed in LDS
    __syncthreads();    // ... and every wavefront is done with the current one
  };

  using B0 = std::false_type;
  using B1 = std::true_type;
  for (int kb = u0; kb < u1; kb += 2) {
    tile(kb, kb + 1, std::false_type{}, B0{});
    tile(kb + 1, kb + 2 < u1 ? kb + 2 : (n_mask > 0 ? masked_kb(0) : -1), std::false_type{}, B1{});
  }
  int j = 0;
  for (; j + 2 <= n_mask; j += 2) {
    tile(masked_kb(j), masked_kb(j + 1), std::true_type{}, B0{});
    tile(masked_kb(j + 1), j + 2 < n_mask ? masked_kb(j + 2) : -1, std::true_type{}, B1{});
  }
  if (j < n_mask) tile(masked_kb(j), -1, std::true_type{}, B0{});

  // Epilogue.
  const float l_tot = pair_sum(l_run);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = (uint16_t*)a.out + (size_t)(q_start + my_row) * q_rs + (size_t)h * Dr;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = d * 32 + 8 * g + 4 * lh;
        u32x2 w;
        w.x = pack2<BF16>(acc[d][4 * g + 0] * inv, acc[d][4 * g + 1] * inv);
        w.y = pack2<BF16>(acc[d][4 * g + 2] * inv, acc[d][4 * g + 3] * inv);
        if (col < Dr) *(u32x2*)(op + col) = w;  // four columns, all inside or all past Dr
      }
    }
    if (lh == 0) {
      float lse = INFINITY;
      if (l_tot > 0.f) lse = (ALIBI ? m_run * 0.69314718055994531f : m_run * a.scale) + __logf(l_tot);
      size_t idx;
      if constexpr (VARLEN) {
        idx = (size_t)h * load_uniform(a.cu_q + a.B) + q_start + my_row;
      } else {
        idx = ((size_t)b * a.Hq + h) * a.Sq + my_row;
      }
      a.lse[idx] = lse;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Ping-pong forward kernel (D <= 128).
//
// Same arithmetic as fwd_kernel, scheduled so that the matrix pipe stays busy.  On a CDNA4
// SIMD one wavefront issues a VALU instruction only every ~6 cycles while a 32x32x16 MFMA
// holds the matrix pipe for 32 cycles; two wavefronts that run their softmax at the same
// time (and then their products at the same time) leave the pipe idle for about half of
// the loop.  Here a workgroup of 8 wavefronts (256 query rows, 32 per wavefront) splits
// into two groups with one wavefront of each on every SIMD, and workgroup barriers cut the
// loop into phases:
//   M phase of tile j: S^T(j) = K(j) Q^T and O^T += V(j-1)^T P^T(j-1)   (MFMA and LDS reads)
//   X phase of tile j: masking, running max and sum, P(j) = exp2(...), rescale of O
// Group 1 runs one phase behind group 0, so on every SIMD one wavefront multiplies while
// the other runs its softmax.  Both groups execute the same instruction stream (group 1
// only starts one barrier later), which keeps the register allocation that of one path.
//
// Tiles move through LDS in stages: stage s holds K of tile s and V of tile s-1 in
// processing order, in buffer s % 3.  Every wavefront issues its share of stage j+2 among
// the VALU work of X(j) and waits for it at the end of M(j+1), just before the barrier
// after which stage j+2 may be read.  The query rows live in LDS too (each wavefront its
// own 32 rows, read with the same offsets as a K tile), which leaves the registers to the
// accumulators and to operand reads issued a few products ahead.
// How far a row maximum may outgrow the exponent reference (exp2 units) before the
// reference moves and the accumulator is rescaled: probabilities stay below 2^8.
constexpr float kLazyRef = 8.f;
constexpr int kPPWaves = 8;
constexpr int kPPBM = 32 * kPPWaves;  // query rows per workgroup
constexpr int kPPBN = 64;             // keys per tile

template <int D, bool BF16, bool MASKED, bool VARLEN, bool ALIBI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_pp_kernel(FwdArgs a) {
  if (debug_stop(a.dbg)) return;
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int TILE = kPPBN * D;
  using Swz = DualSwizzle<D>;
  // Stage buffers as distinct LDS objects, always addressed statically, so that the
  // compiler can tell operand reads from the direct loads in flight into other buffers.
  __shared__ __attribute__((aligned(16))) uint16_t K0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t K1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t K2[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V2[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[kPPWaves * 32 * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // waves w and w + 4 share a SIMD
  const int li = lane & 31;
  const int lh = lane >> 5;

  int b, h, qb;
  if (!fwd_block<kPPBM, VARLEN>(a, b, h, qb)) return;  // uniform over the workgroup

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
  const int q0 = qb * kPPBM;
  if (q0 >= Lq) return;  // uniform over the workgroup

  const int hk = h / (a.Hq / a.Hkv);
  const int Dr = a.D;  // head dimension of the tensors (<= D, the tile width)
  const int Dc = Dr / 8;
  const size_t q_rs = (size_t)a.Hq * Dr;
  const size_t k_rs = (size_t)a.Hkv * Dr;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)k_start * k_rs + (size_t)hk * Dr;
  const uint16_t* vp = (const uint16_t*)a.v + (size_t)k_start * k_rs + (size_t)hk * Dr;

  const int diag = Lk - Lq;
  KeyWindow kw{Lk, diag, 0, -1, -1};
  if constexpr (MASKED) kw = KeyWindow{Lk, diag, a.causal, a.window_left, a.window_right};
  const int last_row = min(q0 + kPPBM, Lq) - 1;
  const int k_lo = kw.lo(q0), k_hi = kw.hi(last_row);
  const int kb_begin = k_lo / kPPBN;
  const int kb_end = k_hi >= k_lo ? k_hi / kPPBN + 1 : kb_begin;
  const int all_lo = kw.lo(last_row), all_hi = kw.hi(q0);

  const int my_row = q0 + wave * 32 + li;
  const bool row_ok = my_row < Lq;
  const int wave_row0 = q0 + wave * 32;
  const int wave_lo = kw.lo(wave_row0), wave_hi = kw.hi(min(wave_row0 + 31, Lq - 1));
  const int my_lo = kw.lo(my_row), my_hi = kw.hi(my_row);

  // Processing order: the run of tiles every row keeps in full (a multiple of three
  // long, so that the three stage buffers repeat with the loop), then the edge tiles
  // (before the run: window; after it: diagonal, tail).
  const int u0 = min(max(kb_begin, (all_lo + kPPBN - 1) / kPPBN), kb_end);
  int u1 = all_hi >= 0 ? min(kb_end, (all_hi + 1) / kPPBN) : 0;
  u1 = u1 > u0 ? u0 + (u1 - u0) / 3 * 3 : u0;
  const int n_un = u1 - u0;
  const int n_lead = u0 - kb_begin;
  const int n = n_un + n_lead + (kb_end - u1);
  auto kbj = [&](int j) __attribute__((always_inline)) {
    const int i = j - n_un;
    const int edge = i < n_lead ? kb_begin + i : u1 + (i - n_lead);
    return j < n_un ? u0 + j : edge;
  };

  // This wavefront's share of stage st (NI 16-byte chunks per lane of each tile).
  // Indexes past either end repeat a valid tile (the buffer it lands in is free and is
  // not read), so the loads carry no branch and can be scheduled among other work; rows
  // past the end of the sequence re-read the last row (finite data, masked to P = 0).
  constexpr int NI = TILE / 8 / (64 * kPPWaves);
  static_assert(NI >= 1 && (TILE / 8) % (64 * kPPWaves) == 0, "whole chunks per lane");
  // One buffer resource per tensor over this sequence and head (K/V rows of a sequence
  // span less than 4 GiB, which the host checks); a tile's first row goes in the scalar
  // offset, the row and column within the tile in the lane offset.
  const uint32_t krs2 = (uint32_t)k_rs * 2u;
  const size_t kv_first = (size_t)k_start * k_rs + (size_t)hk * Dr;
  const size_t kv_rest = ((size_t)(VARLEN ? load_uniform(a.cu_k + a.B) : a.B * a.Sk) * k_rs - kv_first) * 2u;
  const uint32_t kv_bytes = (uint32_t)(kv_rest < 0xffffffffu ? kv_rest : 0xffffffffu);
  const auto kr = make_rsrc(kp, kv_bytes);
  const auto vr = make_rsrc(vp, kv_bytes);
  // Row and swizzled column (bytes) of this lane's chunks within a tile.
  int lrow[NI];
  uint32_t lcol[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int chunk = (i * kPPWaves + wave) * 64 + lane;
    lrow[i] = chunk / Swz::CH;
    lcol[i] = (uint32_t)(src_chunk(Swz::chunk(lrow[i], chunk % Swz::CH), Dc) * 16);
  }
  // First keys of the K and V tiles of stage st (wavefront-uniform), computed before the
  // M phase that precedes the X phase issuing the loads.
  struct StageSrc {
    int kk0, vk0;
  };
  auto stage_src = [&](int st) __attribute__((always_inline)) {
    // readfirstlane: keep them in scalar registers (the scalar offset of a buffer load).
    return StageSrc{__builtin_amdgcn_readfirstlane(kbj(min(st, n - 1)) * kPPBN),
                    __builtin_amdgcn_readfirstlane(kbj(max(min(st - 1, n - 1), 0)) * kPPBN)};
  };
  auto load_stage = [&](StageSrc src, uint16_t* Kd, uint16_t* Vd) __attribute__((always_inline)) {
    const int klim = Lk - 1 - src.kk0, vlim = Lk - 1 - src.vk0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      // row * row_bytes + column in one 24-bit multiply-add (rows < 64; the host keeps
      // row_bytes below 2^24).
      lds_buffer_load16(kr, __umul24((uint32_t)min(lrow[i], klim), krs2) + lcol[i],
                        Kd + (i * kPPWaves + wave) * 64 * 8, (uint32_t)src.kk0 * krs2);
      lds_buffer_load16(vr, __umul24((uint32_t)min(lrow[i], vlim), krs2) + lcol[i],
                        Vd + (i * kPPWaves + wave) * 64 * 8, (uint32_t)src.vk0 * krs2);
    }
  };
  auto kbuf = [&](auto bi) __attribute__((always_inline)) {
    constexpr int I = decltype(bi)::value % 3;
    return I == 0 ? K0 : (I == 1 ? K1 : K2);
  };
  auto vbuf = [&](auto bi) __attribute__((always_inline)) {
    constexpr int I = decltype(bi)::value % 3;
    return I == 0 ? V0 : (I == 1 ? V1 : V2);
  };

  // Q rows of this wavefront into its LDS region (rows past the end of the sequence
  // re-read the last row; their results are not stored), then stages 0 and 1.
  // A wavefront can lie wholly past the end (q0 < Lq <= wave_row0): rows are clamped as
  // absolute indexes and addressed from a clamped base row, so every offset is >= 0.
  uint16_t* Qw = Qs + wave * 32 * D;
  {
    const int base_row = min(wave_row0, Lq - 1);
    const size_t qfirst = (size_t)(q_start + base_row) * q_rs + (size_t)h * Dr;
    const size_t qrest = ((size_t)(VARLEN ? load_uniform(a.cu_q + a.B) : a.B * a.Sq) * q_rs - qfirst) * 2u;
    const auto qr = make_rsrc((const uint16_t*)a.q + qfirst, (uint32_t)(qrest < 0xffffffffu ? qrest : 0xffffffffu));
#pragma unroll
    for (int i = 0; i < 32 * D / 8 / 64; ++i) {
      const int chunk = i * 64 + lane;
      const int r = chunk / Swz::CH;
      const int row = min(wave_row0 + r, Lq - 1) - base_row;
      const int g = Swz::chunk(r, chunk % Swz::CH);
      const uint32_t off = (uint32_t)(row * (int)q_rs + g * 8) * 2u;
      if (g < Dc) {
        lds_buffer_load16(qr, off, Qw + i * 64 * 8);
      } else {
        store16(Qw + (i * 64 + lane) * 8, u32x4{0, 0, 0, 0});  // past the head dimension
      }
    }
  }
  if (n > 0) {
    load_stage(stage_src(0), K0, V0);
    load_stage(stage_src(1), K1, V1);
  }

  f32x16 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = f32x16{};
  float m_run = -INFINITY;  // exponent reference of this lane's row (exp2 units / c)
  float l_run = 0.f;        // sum of the probabilities in fp32 (for the LSE)
  float lr_run = 0.f;       // sum of the same probabilities rounded to 16 bits (for O)
  const float c = a.scale_log2;
  constexpr float kLog2e = 1.4426950408889634f;
  float sl2 = 0.f;
  if constexpr (ALIBI) sl2 = a.alibi[(size_t)b * a.alibi_bstride + h] * kLog2e;
  const int row_diag = my_row + diag;

  const int tr_row = 4 * lh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int koff[NS], voff[2][ND];
#pragma unroll
  for (int st = 0; st < NS; ++st) koff[st] = Swz::row_elem(li, st * 2 + lh);
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int d = 0; d < ND; ++d) voff[hi][d] = Swz::elem(tr_row + 8 * hi, d * 32 + tr_col);

  f32x16 s[2];           // S^T of the current tile: M phase -> X phase
  Frag8 pf[4];           // P^T of the previous tile: X phase -> next M phase
  bool pv_live = false;  // pf holds probabilities to add
  // D = 128: lazy exponent reference (kLazyRef), the accumulator rescaled in the X phase
  // when the reference moves, O divided by the sum of the rounded P.  D = 64: the reference
  // follows every new row maximum and the rescale goes into the next M phase, among its
  // S^T products (that phase has half the products of the X phase's length and room for
  // the multiplies; with the lazy reference the extra row sum cost more than it saved
  // there), O divided by the fp32 sum.  Multiplying by exactly 1.0f changes nothing.
  constexpr bool kLazy = D > 64;
  constexpr bool kRescaleInM = !kLazy;
  float alpha_p = 1.f;  // kRescaleInM: rescale of the accumulator due before that product

  // M phase on stage buffer BI: S^T(j) (when the tile is live for this wavefront) and the
  // P V product of the previous tile.  Alone on the matrix pipe, the wavefront has to hide
  // its own LDS latency: the scheduling groups issue the operand reads a few products
  // ahead.
  auto s_part = [&](const uint16_t* K) __attribute__((always_inline)) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      Frag8 qf;
      qf.v = load16(Qw + koff[st]);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        Frag8 kf;
        kf.v = load16(K + sub * 32 * D + koff[st]);
        s[sub] = mfma32x32x16<BF16>(kf, qf, s[sub]);
      }
    }
  };
  auto pv_part = [&](const uint16_t* V) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const u32x2 lo = lds_read_tr16(V + t * 16 * D + voff[0][d]);
        const u32x2 hi = lds_read_tr16(V + t * 16 * D + voff[1][d]);
        Frag8 vf;
        vf.v = u32x4{lo.x, lo.y, hi.x, hi.y};
        acc[d] = mfma32x32x16<BF16>(vf, pf[t], acc[d]);
      }
    }
  };
  // Operand reads spread over NM products: R0 issued ahead, the rest evenly over all
  // but the last two products.
  // NV VALU instructions (the rescale of the accumulator) go four after each of the first
  // NV / 4 products.
  auto read_schedule = [&](auto nm_tag, auto nr_tag, auto id_tag, auto nv_tag) __attribute__((always_inline)) {
    constexpr int NM = decltype(nm_tag)::value, NR = decltype(nr_tag)::value, ID = decltype(id_tag)::value;
    constexpr int NV = decltype(nv_tag)::value;
    constexpr int R0 = NR < 8 ? NR : 8, RR = NR - R0, SL = NM - 2;
    __builtin_amdgcn_sched_group_barrier(0x100, R0, ID);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);
      const int cnt = i < SL ? (i + 1) * RR / SL - i * RR / SL : 0;
#pragma unroll
      for (int k = 0; k < cnt; ++k) __builtin_amdgcn_sched_group_barrier(0x100, 1, ID);
      if (i < NV / 4) __builtin_amdgcn_sched_group_barrier(0x002, 4, ID);
    }
  };

  // M phase on stage buffer BI: S^T(j) (when the tile is live for this wavefront) and the
  // P V product of the previous tile.  Alone on the matrix pipe, the wavefront has to hide
  // its own LDS latency, so the operand reads are issued several products ahead; when
  // both products are certain (FUSED: interior tiles after the first) they form one block
  // and share one read schedule.
  auto mphase = [&](bool s_live, auto bi, auto fused_tag) __attribute__((always_inline)) {
    constexpr bool FUSED = decltype(fused_tag)::value;
    const uint16_t* K = kbuf(bi);
    const uint16_t* V = vbuf(bi);
    if constexpr (FUSED) {
      s_part(K);
      if constexpr (kRescaleInM) {
#pragma unroll
        for (int d = 0; d < ND; ++d) acc[d] *= alpha_p;
      }
      pv_part(V);
      read_schedule(Idx<2 * NS + 4 * ND>{}, Idx<3 * NS + 8 * ND>{}, Idx<0>{}, Idx<kRescaleInM ? 16 * ND : 0>{});
    } else {
      if (s_live) {
        s_part(K);
        read_schedule(Idx<2 * NS>{}, Idx<3 * NS>{}, Idx<0>{}, Idx<0>{});
      }
      if (pv_live) {
        if constexpr (kRescaleInM) {
#pragma unroll
          for (int d = 0; d < ND; ++d) acc[d] *= alpha_p;
        }
        pv_part(V);
        read_schedule(Idx<4 * ND>{}, Idx<8 * ND>{}, Idx<1>{}, Idx<0>{});
      }
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) pin(s[sub]);
#pragma unroll
    for (int d = 0; d < ND; ++d) pin(acc[d]);
  };

  // X phase of the tile at key k0; first issues this wavefront's share of stage st_next
  // into buffer BI, spread among the softmax arithmetic.
  auto xphase = [&](int k0, bool live, auto mask_tag, StageSrc next, auto bi) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    load_stage(next, kbuf(bi), vbuf(bi));
    pv_live = live;
    alpha_p = 1.f;
    if (!live) return;
    if constexpr (ALIBI) {
      const float base = (float)(k0 + 4 * lh - row_diag);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float dist = base + (float)(sub * 32 + 8 * (r >> 2) + (r & 3));
          s[sub][r] = fmaf(-sl2, fabsf(dist), s[sub][r] * c);
        }
    }
    if constexpr (MASK) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + sub * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          s[sub][r] = (key >= my_lo && key <= my_hi) ? s[sub][r] : -INFINITY;
        }
    }
    float mx = m_run;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
    mx = pair_max(mx);
    // kLazy: the exponent reference m_run moves only when the row maximum outgrows it by
    // more than kLazyRef (exp2 units), or from -inf at the row's first kept key; otherwise
    // the probabilities stay relative to it (at most 2^kLazyRef) and the accumulator
    // needs no rescale.  (Both sides -inf: NaN compares false, the row stays empty.)
    // Otherwise the reference is the running row maximum itself.
    float m_use, alpha = 1.f;
    if constexpr (kLazy) {
      const bool move = (ALIBI ? mx - m_run : (mx - m_run) * c) > kLazyRef;
      const float m_new = move ? mx : m_run;
      m_use = (m_new == -INFINITY) ? 0.f : m_new;
      if (move) alpha = ALIBI ? fast_exp2(m_run - m_use) : (m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_use) * c));
      m_run = m_new;
    } else {
      m_use = (mx == -INFINITY) ? 0.f : mx;
      alpha = ALIBI ? fast_exp2(m_run - m_use) : (m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_use) * c));
      m_run = mx;
    }
    float ls = 0.f;
    if constexpr (ALIBI) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(s[sub][r] - m_use);
          s[sub][r] = p;
          ls += p;
        }
    } else {
      const float mc = m_use * c;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[sub][r], c, -mc));
          s[sub][r] = p;
          ls += p;
        }
    }
    if constexpr (!MASK) {
      // Spread the direct loads over the softmax arithmetic.
#pragma unroll
      for (int i = 0; i < 2 * NI; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 2);
        __builtin_amdgcn_sched_group_barrier(0x002, 20, 2);
      }
    }
    l_run = l_run * alpha + ls;
    if constexpr (kRescaleInM) {
      alpha_p = alpha;  // applied to the accumulator in the next M phase
    } else if (__builtin_expect(__any(alpha != 1.f), 0)) {
#pragma unroll
      for (int d = 0; d < ND; ++d) acc[d] *= alpha;
    }
    float lrs = 0.f;  // sum of the rounded probabilities, the weights the P V product uses
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int sub = t >> 1, r0 = (t & 1) * 8;
      pf[t].v = u32x4{pack2<BF16>(s[sub][r0 + 0], s[sub][r0 + 1]), pack2<BF16>(s[sub][r0 + 2], s[sub][r0 + 3]),
                      pack2<BF16>(s[sub][r0 + 4], s[sub][r0 + 5]), pack2<BF16>(s[sub][r0 + 6], s[sub][r0 + 7])};
      if constexpr (kLazy) {
#pragma unroll
        for (int w = 0; w < 4; ++w) lrs = sum2<BF16>(pf[t].v[w], lrs);
      }
      pin(pf[t].v);
    }
    if constexpr (kLazy) lr_run = lr_run * alpha + lrs;
    if constexpr (kRescaleInM) {
      pin(alpha_p);
    } else {
#pragma unroll
      for (int d = 0; d < ND; ++d) pin(acc[d]);
    }
    pin(m_run);
    pin(l_run);
    if constexpr (kLazy) pin(lr_run);
  };

  // Tile j of the processing order, stage buffer BI = j % 3.  The wait at the end of the
  // M phase covers the stage this wavefront issued in the previous X phase.
  auto step = [&](int j, auto mask_tag, auto bi, auto fused_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int BI = decltype(bi)::value;
    const int k0 = kbj(j) * kPPBN;
    const bool live = !MASK || !(k0 > wave_hi || k0 + kPPBN - 1 < wave_lo);
    const StageSrc next = stage_src(j + 2);
    mphase(live, bi, fused_tag);
    wait_vmcnt<0>();
    phase_barrier();
    xphase(k0, live, mask_tag, next, Idx<BI + 2>{});
    phase_barrier();
  };

  // Q and stage 0 have landed (stage 1, issued last, may still be in flight: the wait at
  // the end of the first M phase covers it), everywhere after the barrier.
  if (n > 0) {
    wait_vmcnt<2 * NI>();
  } else {
    wait_vmcnt<0>();
  }
  lds_barrier();
  if (grp == 1) phase_barrier();
  using F = std::false_type;
  using T = std::true_type;
  // Interior tiles; the first one has no previous tile to add.
  if (n_un > 0) {
    step(0, F{}, Idx<0>{}, F{});
    step(1, F{}, Idx<1>{}, T{});
    step(2, F{}, Idx<2>{}, T{});
  }
  for (int j = 3; j < n_un; j += 3) {
    step(j, F{}, Idx<0>{}, T{});
    step(j + 1, F{}, Idx<1>{}, T{});
    step(j + 2, F{}, Idx<2>{}, T{});
  }
  // Edge tiles.
  int j = n_un;
  for (; j + 3 <= n; j += 3) {
    step(j, T{}, Idx<0>{}, F{});
    step(j + 1, T{}, Idx<1>{}, F{});
    step(j + 2, T{}, Idx<2>{}, F{});
  }
  if (j < n) step(j, T{}, Idx<0>{}, F{});
  if (j + 1 < n) step(j + 1, T{}, Idx<1>{}, F{});
  // Last M phase: the P V product of the last tile (stage n, buffer n % 3).
  const int nb = n % 3;
  if (nb == 0) {
    mphase(false, Idx<0>{}, F{});
  } else if (nb == 1) {
    mphase(false, Idx<1>{}, F{});
  } else {
    mphase(false, Idx<2>{}, F{});
  }
  wait_vmcnt<0>();  // the last X phase's loads (repeats of valid tiles) have landed
  if (grp == 0) phase_barrier();

  const float l_tot = pair_sum(l_run);
  const float lr_tot = kLazy ? pair_sum(lr_run) : 0.f;
  {
    // kLazy: O is normalised by the sum of the weights its product used (the rounded P),
    // so that one dominant key yields exactly its value however far the reference lags.
    const float den = kLazy ? lr_tot : l_tot;
    const float inv = den > 0.f ? 1.f / den : 0.f;
    // The rows go out whole: through this wavefront's Q region of LDS (no longer read;
    // 16-byte chunk c of row r at chunk c ^ (r % CH), so that neither the 8-byte writes of a
    // column group nor the 16-byte row reads pile onto a few banks), then 16 bytes per lane
    // with CH lanes per row.  Stored directly, a lane's four columns made every store
    // instruction touch 32 rows; this way one touches 64 / CH.
    constexpr int CH = D / 8;
    // lane-derived offsets recomputed here rather than kept live through the loops
    const int ln = opaque(lane), lr = ln & 31, lc = ln >> 5;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w.x = pack2<BF16>(acc[d][4 * g + 0] * inv, acc[d][4 * g + 1] * inv);
        w.y = pack2<BF16>(acc[d][4 * g + 2] * inv, acc[d][4 * g + 3] * inv);
        *(u32x2*)(Qw + lr * D + (((4 * d + g) ^ (lr % CH)) * 8) + 4 * lc) = w;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const int rows_in = Lq - wave_row0;  // this wavefront's rows inside the sequence
    const size_t obase = (size_t)(q_start + wave_row0) * q_rs + (size_t)h * Dr;
    const size_t ototal = (size_t)(VARLEN ? load_uniform(a.cu_q + a.B) : a.B * a.Sq) * q_rs;
    const auto orr = make_rsrc((const uint16_t*)a.out + obase, bytes_left(ototal, obase, 2u));
#pragma unroll
    for (int i = 0; i < 32 * CH / 64; ++i) {
      const int r = (i * 64 + ln) / CH, c = (i * 64 + ln) % CH;
      const u32x4 v = load16(Qw + r * D + ((c ^ (r % CH)) * 8));
      if (r < rows_in && c * 8 < Dr) buffer_store16(orr, (uint32_t)(r * (int)q_rs + c * 8) * 2u, v);
    }
  }
  if (row_ok) {
    if (lh == 0) {
      float lse = INFINITY;
      if (l_tot > 0.f) lse = (ALIBI ? m_run * 0.69314718055994531f : m_run * a.scale) + __logf(l_tot);
      size_t idx;
      if constexpr (VARLEN) {
        idx = (size_t)h * load_uniform(a.cu_q + a.B) + q_start + my_row;
      } else {
        idx = ((size_t)b * a.Hq + h) * a.Sq + my_row;
      }
      a.lse[idx] = lse;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Key-split ping-pong forward kernel (D = 256).
//
// The ping-pong schedule of fwd_pp_kernel needs two wavefronts per SIMD; at D = 256 the
// output accumulator alone takes 128 registers per lane, and 256 query rows of Q (128 KiB)
// do not fit in LDS beside the tile stages.  Here the two wavefronts of a SIMD work on the
// SAME 32 query rows and split the keys instead: group 0 takes the even tiles of the
// processing order, group 1 the odd ones, each with its own running max, sum and
// accumulator.  A workgroup is 128 query rows (four SIMD pairs) and its Q takes 64 KiB of
// LDS.  Tiles are 32 keys, so the X phase handles half as many scores per wavefront as
// at D = 128 while the M phase has the same 32 products: the matrix pipe, not the softmax,
// sets the period.  At the end the two partial softmax states of each row are merged
// (the rule of the online softmax: rescale both to the larger max and add), through LDS.
//
// Items (one K tile and one V tile each) are consumed in interval order: item k is read by
// the M phase of group k % 2 at interval k and holds K of tile k and V of tile k - 2 (the
// P V product of that group's previous tile).  Item k lives in buffer k % 3: the X phase
// right after a group read item k loads item k + 3 into the same buffer, and the group
// waits for it at the end of its next M phase, before the barrier after which item k + 3
// is read.
constexpr int kKPWaves = 8;
constexpr int kKPBM = 32 * (kKPWaves / 2);  // query rows per workgroup
constexpr int kKPBN = 32;                   // keys per tile

template <bool BF16, bool MASKED, bool VARLEN, bool ALIBI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kp_kernel(FwdArgs a) {
  if (debug_stop(a.dbg)) return;
  constexpr int D = 256;
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int TILE = kKPBN * D;
  using Swz = DualSwizzle<D>;
  __shared__ __attribute__((aligned(16))) uint16_t K0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t K1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t K2[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V2[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[(kKPWaves / 2) * 32 * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // waves w and w + 4 share a SIMD and their query rows
  const int pr = wave & 3;    // the pair: rows 32 pr .. 32 pr + 31 of the block
  const int li = lane & 31;
  const int lh = lane >> 5;

  int b, h, qb;
  if (!fwd_block<kKPBM, VARLEN>(a, b, h, qb)) return;  // uniform over the workgroup

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
  const int q0 = qb * kKPBM;
  if (q0 >= Lq) return;  // uniform over the workgroup

  const int hk = h / (a.Hq / a.Hkv);
  const int Dr = a.D;  // head dimension of the tensors (<= D, the tile width)
  const int Dc = Dr / 8;
  const size_t q_rs = (size_t)a.Hq * Dr;
  const size_t k_rs = (size_t)a.Hkv * Dr;
  const uint16_t* kp = (const uint16_t*)a.k + (size_t)k_start * k_rs + (size_t)hk * Dr;
  const uint16_t* vp = (const uint16_t*)a.v + (size_t)k_start * k_rs + (size_t)hk * Dr;

  const int diag = Lk - Lq;
  KeyWindow kw{Lk, diag, 0, -1, -1};
  if constexpr (MASKED) kw = KeyWindow{Lk, diag, a.causal, a.window_left, a.window_right};
  const int last_row = min(q0 + kKPBM, Lq) - 1;
  const int k_lo = kw.lo(q0), k_hi = kw.hi(last_row);
  const int kb_begin = k_lo / kKPBN;
  const int kb_end = k_hi >= k_lo ? k_hi / kKPBN + 1 : kb_begin;
  const int all_lo = kw.lo(last_row), all_hi = kw.hi(q0);

  const int wave_row0 = q0 + pr * 32;
  const int my_row = wave_row0 + li;
  const bool row_ok = my_row < Lq;
  const int wave_lo = kw.lo(wave_row0), wave_hi = kw.hi(min(wave_row0 + 31, Lq - 1));
  const int my_lo = kw.lo(my_row), my_hi = kw.hi(my_row);

  // Processing order: the run of tiles every row keeps in full (a multiple of six long,
  // so that each group's steps repeat the three buffers with the loop), then the edge
  // tiles (before the run: window; after it: diagonal, tail).
  const int u0 = min(max(kb_begin, (all_lo + kKPBN - 1) / kKPBN), kb_end);
  int u1 = all_hi >= 0 ? min(kb_end, (all_hi + 1) / kKPBN) : 0;
  u1 = u1 > u0 ? u0 + (u1 - u0) / 6 * 6 : u0;
  const int n_un = u1 - u0;
  const int n_lead = u0 - kb_begin;
  const int n = n_un + n_lead + (kb_end - u1);
  auto kbj = [&](int j) __attribute__((always_inline)) {
    const int i = j - n_un;
    const int edge = i < n_lead ? kb_begin + i : u1 + (i - n_lead);
    return j < n_un ? u0 + j : edge;
  };
  const int n_s = (n + 1) / 2;  // steps per group; group 1's last one is empty when n is odd
  const int s_un = n_un / 2;    // interior steps per group, a multiple of three

  // An item is loaded by the four wavefronts of one group: NI 16-byte chunks per lane of
  // each tile.  Indexes past either end repeat a valid tile (its buffer is free and is not
  // read); rows past the end of the sequence re-read the last row (finite, masked to 0).
  constexpr int NI = TILE / 8 / (64 * 4);
  static_assert(NI >= 1 && (TILE / 8) % (64 * 4) == 0, "whole chunks per lane");
  const uint32_t krs2 = (uint32_t)k_rs * 2u;
  const size_t kv_first = (size_t)k_start * k_rs + (size_t)hk * Dr;
  const size_t kv_rest = ((size_t)(VARLEN ? load_uniform(a.cu_k + a.B) : a.B * a.Sk) * k_rs - kv_first) * 2u;
  const uint32_t kv_bytes = (uint32_t)(kv_rest < 0xffffffffu ? kv_rest : 0xffffffffu);
  const auto kr = make_rsrc(kp, kv_bytes);
  const auto vr = make_rsrc(vp, kv_bytes);
  // Row and swizzled column (bytes) of this lane's chunk i of a tile.
  auto lrow = [&](int i) __attribute__((always_inline)) { return ((i * 4 + pr) * 64 + lane) / Swz::CH; };
  auto lcol = [&](int i) __attribute__((always_inline)) {
    return (uint32_t)(src_chunk(Swz::chunk(lrow(i), lane % Swz::CH), Dc) * 16);
  };
  uint32_t loff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) loff[i] = __umul24((uint32_t)lrow(i), krs2) + lcol(i);
  struct ItemSrc {
    int kk0, vk0;
  };
  auto item_src = [&](int k) __attribute__((always_inline)) {
    return ItemSrc{__builtin_amdgcn_readfirstlane(kbj(min(k, n - 1)) * kKPBN),
                   __builtin_amdgcn_readfirstlane(kbj(max(min(k - 2, n - 1), 0)) * kKPBN)};
  };
  auto load_item = [&](ItemSrc src, uint16_t* Kd, uint16_t* Vd) __attribute__((always_inline)) {
    if (max(src.kk0, src.vk0) + kKPBN <= Lk) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        lds_buffer_load16(kr, loff[i], Kd + (i * 4 + pr) * 64 * 8, (uint32_t)src.kk0 * krs2);
        lds_buffer_load16(vr, loff[i], Vd + (i * 4 + pr) * 64 * 8, (uint32_t)src.vk0 * krs2);
      }
    } else {
      // A tile that runs past the last key: clamp its rows (rows < 32; the host keeps
      // row_bytes below 2^24 for the 24-bit multiply).
      const int klim = Lk - 1 - src.kk0, vlim = Lk - 1 - src.vk0;
      const int ln = opaque(lane);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = ((i * 4 + pr) * 64 + ln) / Swz::CH;
        const uint32_t col = (uint32_t)(src_chunk(Swz::chunk(row, ln % Swz::CH), Dc) * 16);
        lds_buffer_load16(kr, __umul24((uint32_t)min(row, klim), krs2) + col, Kd + (i * 4 + pr) * 64 * 8,
                          (uint32_t)src.kk0 * krs2);
        lds_buffer_load16(vr, __umul24((uint32_t)min(row, vlim), krs2) + col, Vd + (i * 4 + pr) * 64 * 8,
                          (uint32_t)src.vk0 * krs2);
      }
    }
  };
  auto kbuf = [&](auto bi) __attribute__((always_inline)) {
    constexpr int I = decltype(bi)::value % 3;
    return I == 0 ? K0 : (I == 1 ? K1 : K2);
  };
  auto vbuf = [&](auto bi) __attribute__((always_inline)) {
    constexpr int I = decltype(bi)::value % 3;
    return I == 0 ? V0 : (I == 1 ? V1 : V2);
  };

  // Q rows of the pair into its LDS region, split between its two wavefronts (rows past
  // the end re-read the last row, clamped as absolute indexes from a clamped base row),
  // then items 0 and 2 by group 0, item 1 by group 1.
  uint16_t* Qw = Qs + pr * 32 * D;
  {
    const int base_row = min(wave_row0, Lq - 1);
    const size_t qfirst = (size_t)(q_start + base_row) * q_rs + (size_t)h * Dr;
    const size_t qrest = ((size_t)(VARLEN ? load_uniform(a.cu_q + a.B) : a.B * a.Sq) * q_rs - qfirst) * 2u;
    const auto qr = make_rsrc((const uint16_t*)a.q + qfirst, (uint32_t)(qrest < 0xffffffffu ? qrest : 0xffffffffu));
#pragma unroll
    for (int i = 0; i < 32 * D / 8 / 128; ++i) {
      const int chunk = (i * 2 + grp) * 64 + lane;
      const int r = chunk / Swz::CH;
      const int row = min(wave_row0 + r, Lq - 1) - base_row;
      const int g = Swz::chunk(r, chunk % Swz::CH);
      const uint32_t off = (uint32_t)(row * (int)q_rs + g * 8) * 2u;
      if (g < Dc) {
        lds_buffer_load16(qr, off, Qw + (i * 2 + grp) * 64 * 8);
      } else {
        store16(Qw + ((i * 2 + grp) * 64 + lane) * 8, u32x4{0, 0, 0, 0});  // past the head dimension
      }
    }
  }
  if (n > 0) {
    if (grp == 0) {
      load_item(item_src(0), K0, V0);
      load_item(item_src(2), K2, V2);
    } else {
      load_item(item_src(1), K1, V1);
    }
  }

  f32x16 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = f32x16{};
  float m_run = -INFINITY;  // exponent reference of this lane's row (exp2 units / c)
  float l_run = 0.f;        // sum of the probabilities in fp32 (for the LSE)
  float lr_run = 0.f;       // sum of the same probabilities rounded to 16 bits (for O)
  const float c = a.scale_log2;
  constexpr float kLog2e = 1.4426950408889634f;
  float sl2 = 0.f;
  if constexpr (ALIBI) sl2 = a.alibi[(size_t)b * a.alibi_bstride + h] * kLog2e;
  const int row_diag = my_row + diag;

  // Row reads (row li, chunk 2 st + lh) and transposed reads (rows tr_row + 8 hi, column
  // 32 d + tr_col) of a tile, formed from one base each: with f = f(row) < 16 the swizzled
  // chunk (2 st + lh) ^ f is 2 (st ^ (f >> 1)) + (lh ^ (f & 1)), so the element offset is
  // kbase ^ 16 st; likewise (4 d + c) ^ f = 4 (d ^ (f >> 2)) + (c ^ (f & 3)) for c < 4
  // gives vbase ^ 32 d.  The XOR touches only bits below 256 = D, where the bases hold
  // the row's swizzle; the second half of either range is the first plus 128 (bit 7 of
  // the base is clear), which the reads take as an immediate offset.
  const int tr_row = 4 * lh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int kbase = Swz::row_elem(li, lh);
  int vbase[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) vbase[hi] = Swz::elem(tr_row + 8 * hi, tr_col);

  f32x16 s;              // S^T of the current tile: M phase -> X phase
  Frag8 pf[2];           // P^T of the previous tile: X phase -> next M phase
  bool pv_live = false;  // pf holds probabilities to add

  // The read offsets are re-formed in every M phase from opaque copies of the bases
  // (taken before the phase's reads, so that they do not split its schedule) rather than
  // hoisted into registers that would stay live across the loop.
  // M phase: S^T of this step's tile (when live for this wavefront) and the P V product
  // of the group's previous tile, both from the item this step reads, as one sequence of
  // products: ops 0..NS-1 form S^T (K and Q row reads), ops NS..NS+2ND-1 the P V product
  // (16-key chunk t, d-block d; two transposed V reads).  The operand reads run PD ops
  // ahead, written out in that order and fenced for the machine scheduler, which would
  // otherwise sink each read down to its product.
  constexpr int NOPS = NS + 2 * ND;
  constexpr int PD = 4;
  auto mphase = [&](bool s_live, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, auto fused_tag)
                    __attribute__((always_inline)) {
    constexpr bool FUSED = decltype(fused_tag)::value;
    const int kb = opaque(kbase), vb0 = opaque(vbase[0]), vb1 = opaque(vbase[1]);
    Frag8 opa[PD], opb[PD];
    auto issue = [&](auto op_tag) __attribute__((always_inline)) {
      constexpr int OP = decltype(op_tag)::value, SL = OP % PD;
      if constexpr (OP < NS) {
        const int o = (kb ^ (16 * (OP % (NS / 2)))) + 128 * (OP / (NS / 2));
        opb[SL].v = load16(Qw + o);
        opa[SL].v = load16(K + o);
      } else {
        constexpr int t = (OP - NS) / ND, d = (OP - NS) % ND;
        const int o0 = (vb0 ^ (32 * (d % (ND / 2)))) + 128 * (d / (ND / 2));
        const int o1 = (vb1 ^ (32 * (d % (ND / 2)))) + 128 * (d / (ND / 2));
        const u32x2 lo = lds_read_tr16(V + t * 16 * D + o0);
        const u32x2 hi = lds_read_tr16(V + t * 16 * D + o1);
        opa[SL].v = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    };
    auto run = [&](auto op_tag) __attribute__((always_inline)) {
      constexpr int OP = decltype(op_tag)::value, SL = OP % PD;
      if constexpr (OP < NS) {
        s = mfma32x32x16<BF16>(opa[SL], opb[SL], s);
      } else {
        constexpr int t = (OP - NS) / ND, d = (OP - NS) % ND;
        acc[d] = mfma32x32x16<BF16>(opa[SL], pf[t], acc[d]);
      }
    };
    // Ops [B, E) as one pipeline.
    auto pipeline = [&](auto b_tag, auto e_tag) __attribute__((always_inline)) {
      constexpr int B = decltype(b_tag)::value, E = decltype(e_tag)::value;
      static_for<B, (B + PD < E ? B + PD : E)>([&](auto op) { issue(op); });
      static_for<B, E>([&](auto op) {
        __builtin_amdgcn_sched_barrier(0);  // keep the written order
        run(op);
        constexpr int NX = decltype(op)::value + PD;
        if constexpr (NX < E) issue(Idx<NX>{});
      });
      __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (FUSED) {
      s = f32x16{};
      pipeline(Idx<0>{}, Idx<NOPS>{});
    } else {
      if (s_live) {
        s = f32x16{};
        pipeline(Idx<0>{}, Idx<NS>{});
      }
      if (pv_live) pipeline(Idx<NS>{}, Idx<NOPS>{});
    }
    pin(s);
#pragma unroll
    for (int d = 0; d < ND; ++d) pin(acc[d]);
  };

  // X phase of the tile at key k0; first issues the next item into the buffer the M phase
  // just read.
  auto xphase = [&](int k0, bool live, auto mask_tag, ItemSrc next, uint16_t* __restrict__ Kd,
                    uint16_t* __restrict__ Vd) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    load_item(next, Kd, Vd);
    pv_live = live;
    if (!live) return;
    if constexpr (ALIBI) {
      const float base = (float)(k0 + 4 * lh - row_diag);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dist = base + (float)(8 * (r >> 2) + (r & 3));
        s[r] = fmaf(-sl2, fabsf(dist), s[r] * c);
      }
    }
    if constexpr (MASK) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * lh + (r & 3);
        s[r] = (key >= my_lo && key <= my_hi) ? s[r] : -INFINITY;
      }
    }
    float mx = m_run;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = pair_max(mx);
    // Lazy exponent reference, as in the ping-pong kernel: it moves only when the row
    // maximum outgrows it by more than kLazyRef (exp2 units) or leaves -inf.
    const bool move = (ALIBI ? mx - m_run : (mx - m_run) * c) > kLazyRef;
    const float m_new = move ? mx : m_run;
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    float alpha = 1.f;
    float ls = 0.f;
    if constexpr (ALIBI) {
      if (move) alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(s[r] - m_use);
        s[r] = p;
        ls += p;
      }
    } else {
      if (move) alpha = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_use) * c);
      m_run = m_new;
      const float mc = m_use * c;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[r], c, -mc));
        s[r] = p;
        ls += p;
      }
    }
    l_run = l_run * alpha + ls;
    if (__builtin_expect(__any(alpha != 1.f), 0)) {
#pragma unroll
      for (int d = 0; d < ND; ++d) acc[d] *= alpha;
    }
    float lrs = 0.f;  // sum of the rounded probabilities, the weights the P V product uses
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r0 = t * 8;
      pf[t].v = u32x4{pack2<BF16>(s[r0 + 0], s[r0 + 1]), pack2<BF16>(s[r0 + 2], s[r0 + 3]),
                      pack2<BF16>(s[r0 + 4], s[r0 + 5]), pack2<BF16>(s[r0 + 6], s[r0 + 7])};
#pragma unroll
      for (int w = 0; w < 4; ++w) lrs = sum2<BF16>(pf[t].v[w], lrs);
      pin(pf[t].v);
    }
    lr_run = lr_run * alpha + lrs;
#pragma unroll
    for (int d = 0; d < ND; ++d) pin(acc[d]);
    pin(m_run);
    pin(l_run);
    pin(lr_run);
  };

  // Step i of this group: tile j = 2 i + grp of the processing order, item j, buffer
  // j % 3 = (2 U + grp) % 3 with U = i % 3 (group 0 walks buffers 0, 2, 1, group 1 walks
  // 1, 0, 2).  Both buffer choices are selects on the same condition, so the compiler can
  // still tell the loads in flight from the reads of the next step.
  auto step = [&](int i, auto mask_tag, auto u, auto fused_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int U = decltype(u)::value;
    const int j = 2 * i + grp;
    const int k0 = kbj(min(j, n - 1)) * kKPBN;
    bool live = true;
    if constexpr (MASK) live = j < n && !(k0 > wave_hi || k0 + kKPBN - 1 < wave_lo);
    const ItemSrc next = item_src(j + 3);
    uint16_t* Kc = grp ? kbuf(Idx<2 * U + 1>{}) : kbuf(Idx<2 * U>{});
    uint16_t* Vc = grp ? vbuf(Idx<2 * U + 1>{}) : vbuf(Idx<2 * U>{});
    mphase(live, Kc, Vc, fused_tag);
    wait_vmcnt<0>();
    phase_barrier();
    xphase(k0, live, mask_tag, next, Kc, Vc);
    phase_barrier();
  };

  // Q and each group's first item have landed, everywhere after the barrier (group 0's
  // item 2, issued last, may still be in flight: the wait at the end of its first M phase
  // covers it).
  if (n > 0 && grp == 0) {
    wait_vmcnt<2 * NI>();
  } else {
    wait_vmcnt<0>();
  }
  lds_barrier();
  if (grp == 1) phase_barrier();
  using F = std::false_type;
  using T = std::true_type;
  // Interior steps; the first one has no previous tile to add.
  if (s_un > 0) {
    step(0, F{}, Idx<0>{}, F{});
    step(1, F{}, Idx<1>{}, T{});
    step(2, F{}, Idx<2>{}, T{});
  }
  for (int i = 3; i < s_un; i += 3) {
    step(i, F{}, Idx<0>{}, T{});
    step(i + 1, F{}, Idx<1>{}, T{});
    step(i + 2, F{}, Idx<2>{}, T{});
  }
  // Edge steps.
  int i = s_un;
  for (; i + 3 <= n_s; i += 3) {
    step(i, T{}, Idx<0>{}, F{});
    step(i + 1, T{}, Idx<1>{}, F{});
    step(i + 2, T{}, Idx<2>{}, F{});
  }
  if (i < n_s) step(i, T{}, Idx<0>{}, F{});
  if (i + 1 < n_s) step(i + 1, T{}, Idx<1>{}, F{});
  // Last M phase: the P V product of the group's last tile (item 2 n_s + grp, buffer
  // (2 n_s + grp) % 3).  One copy of the product block with the buffer picked at run time
  // (three static copies made the register allocator spill the accumulators around
  // their join); the last X phase's loads (repeats of valid tiles) are waited for first,
  // as the compiler cannot tell the picked buffer from theirs.
  wait_vmcnt<0>();
  const int vi = (2 * n_s + grp) % 3;
  mphase(false, K0, vi == 0 ? V0 : (vi == 1 ? V1 : V2), F{});
  if (grp == 0) phase_barrier();

  // Merge the two groups' partial states of each row through LDS (every buffer is free
  // once all wavefronts are past the barrier): group 1 writes its accumulator, max and
  // sum; group 0 rescales both to the larger max, adds, and stores.
  const float l_tot = pair_sum(l_run);
  const float lr_tot = pair_sum(lr_run);
  __syncthreads();
  float* xa;
  float* xb;
  if (pr == 0) {
    xa = (float*)K0;
    xb = (float*)K1;
  } else if (pr == 1) {
    xa = (float*)K2;
    xb = (float*)V0;
  } else if (pr == 2) {
    xa = (float*)V1;
    xb = (float*)V2;
  } else {
    xa = (float*)Qs;
    xb = (float*)Qs + TILE / 2;
  }
  float* xs = (float*)Qs + TILE + pr * 192;  // max, sums of the pair's group-1 wavefront
  if (grp == 1) {
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float* dst = (d < ND / 2 ? xa : xb) + (((d % (ND / 2)) * 4 + g) * 64 + lane) * 4;
        *(f32x4*)dst = f32x4{acc[d][4 * g + 0], acc[d][4 * g + 1], acc[d][4 * g + 2], acc[d][4 * g + 3]};
      }
    xs[lane] = m_run;
    xs[64 + lane] = l_tot;
    xs[128 + lane] = lr_tot;
  }
  __syncthreads();
  if (grp == 1) return;
  const float m1 = xs[lane], l1 = xs[64 + lane], lr1 = xs[128 + lane];
  const float m = fmaxf(m_run, m1);
  float a0 = 0.f, a1 = 0.f;
  if (m != -INFINITY) {
    if constexpr (ALIBI) {
      a0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m);
      a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - m);
    } else {
      a0 = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m) * c);
      a1 = m1 == -INFINITY ? 0.f : fast_exp2((m1 - m) * c);
    }
  }
  const float l_all = l_tot * a0 + l1 * a1;
  const float lr_all = lr_tot * a0 + lr1 * a1;
  {
    // O is normalised by the sum of the weights its products used (the rounded P).
    const float inv = lr_all > 0.f ? 1.f / lr_all : 0.f;
    const float w0 = a0 * inv, w1 = a1 * inv;
    u32x2 pk[ND][4];
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      __builtin_amdgcn_sched_barrier(0);  // one d-block at a time: no hoisted reads
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 o1 = *(const f32x4*)((d < ND / 2 ? xa : xb) + (((d % (ND / 2)) * 4 + g) * 64 + lane) * 4);
        pk[d][g].x = pack2<BF16>(acc[d][4 * g + 0] * w0 + o1[0] * w1, acc[d][4 * g + 1] * w0 + o1[1] * w1);
        pk[d][g].y = pack2<BF16>(acc[d][4 * g + 2] * w0 + o1[2] * w1, acc[d][4 * g + 3] * w0 + o1[3] * w1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // The rows go out whole, through xa (the pair's group-1 accumulator there has been
    // read in full; 16-byte chunk c of row r at chunk c ^ (r % CH)), 16 bytes per lane and
    // CH lanes per row: stored directly, every store instruction touched 32 rows.
    constexpr int CH = D / 8;
    uint16_t* ost = reinterpret_cast<uint16_t*>(xa);
    const int ln = opaque(lane), lr = ln & 31, lc = ln >> 5;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) *(u32x2*)(ost + lr * D + (((4 * d + g) ^ (lr % CH)) * 8) + 4 * lc) = pk[d][g];
    __builtin_amdgcn_sched_barrier(0);
    const int rows_in = Lq - wave_row0;  // this pair's rows inside the sequence
    const size_t obase = (size_t)(q_start + wave_row0) * q_rs + (size_t)h * Dr;
    const size_t ototal = (size_t)(VARLEN ? load_uniform(a.cu_q + a.B) : a.B * a.Sq) * q_rs;
    const auto orr = make_rsrc((const uint16_t*)a.out + obase, bytes_left(ototal, obase, 2u));
#pragma unroll
    for (int i = 0; i < 32 * CH / 64; ++i) {
      const int r = (i * 64 + ln) / CH, c = (i * 64 + ln) % CH;
      const u32x4 v = load16(ost + r * D + ((c ^ (r % CH)) * 8));
      if (r < rows_in && c * 8 < Dr) buffer_store16(orr, (uint32_t)(r * (int)q_rs + c * 8) * 2u, v);
    }
  }
  if (row_ok) {
    if (lh == 0) {
      float lse = INFINITY;
      if (l_all > 0.f) lse = (ALIBI ? m * 0.69314718055994531f : m * a.scale) + __logf(l_all);
      size_t idx;
      if constexpr (VARLEN) {
        idx = (size_t)h * load_uniform(a.cu_q + a.B) + q_start + my_row;
      } else {
        idx = ((size_t)b * a.Hq + h) * a.Sq + my_row;
      }
      a.lse[idx] = lse;
    }
  }
}

template <int D, bool BF16, bool MASKED, bool VARLEN, bool ALIBI>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  // The ping-pong kernels address a sequence's K/V rows with 32-bit byte offsets and a
  // K/V row stride below 2^24 bytes.
  const bool offsets_fit =
      (uint64_t)a.Sk * a.Hkv * a.D * 2u < (1ull << 32) - (1ull << 20) && (uint64_t)a.Hkv * a.D * 2u < (1ull << 24);
  if constexpr (D == 256) {
    if (offsets_fit) {
      const int nqb = (a.Sq + kKPBM - 1) / kKPBM;
      const dim3 grid((unsigned)nqb * a.B * a.Hq);
      hipLaunchKernelGGL((fwd_kp_kernel<BF16, MASKED, VARLEN, ALIBI>), grid, dim3(512), 0, stream, a);
      return hipGetLastError();
    }
  }
  if constexpr (D <= 128) {
    if (a.Sq > kFwdBM && offsets_fit) {
      const int nqb = (a.Sq + kPPBM - 1) / kPPBM;
      const dim3 grid((unsigned)nqb * a.B * a.Hq);
      hipLaunchKernelGGL((fwd_pp_kernel<D, BF16, MASKED, VARLEN, ALIBI>), grid, dim3(512), 0, stream, a);
      return hipGetLastError();
    }
  }
  const int nqb = (a.Sq + kFwdBM - 1) / kFwdBM;
  const dim3 grid((unsigned)nqb * a.B * a.Hq);
  hipLaunchKernelGGL((fwd_kernel<D, BF16, MASKED, VARLEN, ALIBI>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool BF16, bool MASKED>
hipError_t launch_fwd_m(const FwdArgs& a, hipStream_t stream) {
  const bool varlen = a.cu_q != nullptr;
  if (a.alibi != nullptr) {
    return varlen ? launch_fwd_t<D, BF16, MASKED, true, true>(a, stream)
                  : launch_fwd_t<D, BF16, MASKED, false, true>(a, stream);
  }
  return varlen ? launch_fwd_t<D, BF16, MASKED, true, false>(a, stream)
                : launch_fwd_t<D, BF16, MASKED, false, false>(a, stream);
}

template <int D, bool BF16>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  const bool masked = a.causal || a.window_left >= 0 || a.window_right >= 0;
  return masked ? launch_fwd_m<D, BF16, true>(a, stream) : launch_fwd_m<D, BF16, false>(a, stream);
}

template <int D>
hipError_t launch_fwd_dt(const FwdArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_fwd_d<D, true>(a, stream) : launch_fwd_d<D, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  switch (tile_headdim(a.D)) {
    case 64: return launch_fwd_dt<64>(a, stream);
    case 128: return launch_fwd_dt<128>(a, stream);
    case 256: return launch_fwd_dt<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
