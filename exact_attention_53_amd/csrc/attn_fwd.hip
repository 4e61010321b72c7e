// Exact attention forward for gfx950.
//
// Pages cited (by title and section):
//   [SA8]  "ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析" 2.1, A.1 (S, P, O), 1.2-1.3 (stats,
//          inference mode, packed QKV strides)
//   [FAT]  "FlashAttention Triton实现中的内存访问模式优化与寄存器分配策略" 2.2 (one program per query
//          block, Q loaded once, running max/sum in on-chip state), 3 (bank conflicts of
//          column reads of K), 4.2 (deferred normalisation), 5 (special-function cost)
//   [2CTA] "深度学习反向传播优化：2-CTA MMA模式与内存访问优化" 3.2, 6.2 (head/batch swizzle,
//          longest-first order, diagonal-first causal traversal)
//
// Structure.  A workgroup of 4 wavefronts owns FWD_BM = 128 query rows of one (b, h);
// wavefront w owns rows 32w .. 32w+31 and keeps them in registers as the B operand of
// S^T = K Q^T, so each lane owns one query row and its running max / sum.  Two
// workgroups share a CU (<= 256 registers per lane), so one wavefront's softmax
// overlaps another's matrix work.  Key/value tiles of FWD_BN = 64 rows are
// double-buffered in LDS:
//   * K [64 keys][d_qk] row-major in swizzled 128-byte rows, filled by direct
//     global->LDS loads (global_load_lds_dwordx4; the swizzle is applied by choosing
//     which global chunk each lane fetches);
//   * V [64 keys][d_v] the same way; the A operand of O^T += V^T P^T is read
//     column-wise with ds_read_b64_tr_b16, which the swizzle keeps conflict-free (two
//     8-byte transposed reads cost the same LDS cycles as one 16-byte row read).  The
//     key order of those reads matches the accumulator layout of S^T, so P^T feeds
//     the MFMA straight from registers.
// Per tile: S^T (2 x d_qk/16 MFMAs), causal / tail mask on diagonal tiles only, row
// max across the tile (one lane swap), p = 2^(S c - m), l += sum p,
// O^T += V^T P^T (d_v/32 x 4 MFMAs).  The running max m is only raised, and O and l
// only rescaled, when a row's maximum grows by more than 2^8; between raises p <= 2^8.
// The result O = O^T / l and LSE = ln 2 (m + log2 l) do not depend on when m was raised.
// Causal: tiles wholly above the diagonal are never loaded; the diagonal tile(s) come
// first; a wavefront skips tiles that lie wholly above its rows.  With a sliding window
// (query i sees keys i-W+1 .. i) the tiles wholly below the band are never loaded
// either; the band's lower edge is masked on the last tiles, which run after the
// unmasked ones, and a wavefront skips tiles wholly below its rows' windows.
#include <type_traits>

#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn53 {

constexpr int FWD_BM = 128;
constexpr int FWD_BN = 64;
constexpr int FWD_NT = 256;
constexpr float kRescaleThreshold = 8.f;  // log2 units
constexpr float kSumLimit = 256.f;        // 2^kRescaleThreshold

// WIN (with CAUSAL only): sliding window of p.win keys.  ALIBI (with CAUSAL only): the
// linear bias -m_h (i - j) added to the scaled scores.
// SPLIT (non-causal only): one key chunk of p.kv_chunk keys per workgroup, partial
// results to p.part.  BSP: block-sparse map (p.bs): the workgroup visits only the key tiles
// of its query block's live key blocks, in the descending order of p.bs's list.  KBIAS: a
// per-key bias (p.kbias, score units) added to the scores; each tile's 64 values travel
// with its keys into LDS.  DROP: dropout with the query-major keep bits p.drop_rows; the
// row sum takes the undropped p, the product P V the kept ones, the epilogue the
// 1 / (1 - p) factor.
template <class E, int DQK, int DV, bool CAUSAL, bool WIN, bool ALIBI, bool SPLIT = false, bool BSP = false,
          bool KBIAS = false, bool DROP = false>
__global__ __launch_bounds__(FWD_NT, 2) void fwd_kernel(FwdParams p) {
  constexpr int KS = DQK / 16;
  constexpr int NDT = DV / 32;
  constexpr int KT_BYTES = FWD_BN * DQK * 2;
  constexpr int VT_BYTES = FWD_BN * DV * 2;
  // One LDS object per buffer: the compiler can then tell the reads of one buffer
  // from the direct loads in flight into the other and does not wait on them.
  __shared__ __attribute__((aligned(1024))) char kbuf0[KT_BYTES], kbuf1[KT_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[VT_BYTES], vbuf1[VT_BYTES];
  __shared__ __attribute__((aligned(256))) float kbl0[KBIAS ? FWD_BN : 1], kbl1[KBIAS ? FWD_BN : 1];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, lq = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: kept in a scalar register
  const int T = p.T;
  const int nqb = (T + FWD_BM - 1) / FWD_BM;
  // Lq / Lk: valid query / key rows of this batch (T and Tk, or the padded-batch lengths)
  int qb, b, h, Lq = T, Lk = p.Tk;
  const int nbase = nqb * p.B * p.NH;
  const int split = SPLIT ? (int)blockIdx.x / nbase : 0;
  if constexpr (BSP) {  // work list of (b * NH + h, query block), longest first
    const int bhi = p.bs.items[2 * blockIdx.x];
    qb = p.bs.items[2 * blockIdx.x + 1];
    b = bhi / p.NH;
    h = bhi % p.NH;
  } else if (p.items == nullptr) {
    const Item item = schedule(SPLIT ? (int)blockIdx.x % nbase : (int)blockIdx.x, p.B * p.NH);
    qb = CAUSAL ? nqb - 1 - item.rank : item.rank;
    b = item.bh / p.NH;
    h = item.bh % p.NH;
    if (p.seq_k != nullptr) Lk = batch_len(p.seq_k, b, p.Tk);  // decode: per-sequence cache length
  } else {
    const ListItem it = list_item(blockIdx.x, p.NH, p.items);
    b = it.b;
    h = it.h;
    qb = it.blk;
    Lq = batch_len(p.seq_q, b, T);
    Lk = batch_len(p.seq_k, b, T);
  }
  const int bh = b * p.NH + h;

  const E* qg = (const E*)p.q + b * p.sq.b + h * p.sq.h;
  const E* kg = (const E*)p.k + b * p.sk.b + h * p.sk.h;
  const E* vg = (const E*)p.v + b * p.sv.b + h * p.sv.h;
  E* og = (E*)p.o + b * p.so.b + h * p.so.h;
  const int64_t skt = p.sk.t, svt = p.sv.t;

  const LdsLane L = lds_lane(lane);
  const int q0 = qb * FWD_BM;
  const int qw = q0 + 32 * w;
  const int my_q = qw + lq;
  const int W = WIN ? p.win : kNoWindow;
  // key split: this workgroup's keys are [c0, kv_end)
  const int c0 = SPLIT ? split * p.kv_chunk : 0;
  const int kv_end = CAUSAL ? min(Lk, q0 + FWD_BM) : SPLIT ? min(Lk, c0 + p.kv_chunk) : Lk;
  const int n_kv = (kv_end + FWD_BN - 1) / FWD_BN;
  // sliding window: tiles below j_lo hold no key of any row's window
  const int j_lo = WIN ? max(0, q0 - W + 1) / FWD_BN : SPLIT ? c0 / FWD_BN : 0;
  // Block-sparse: the live key blocks (descending) hold two tiles each; the upper tile of
  // the highest one may lie wholly past kv_end and is then left out.
  const int* bs_idx = BSP ? p.bs.idx + ((int64_t)bh * nqb + qb) * p.bs.nb : nullptr;
  const int bs_cnt = BSP ? p.bs.cnt[bh * nqb + qb] : 0;
  const int bs_skip = (BSP && bs_cnt > 0 && bs_idx[0] * kBsBlock + FWD_BN >= kv_end) ? 1 : 0;
  const int n_tiles = BSP ? 2 * bs_cnt - bs_skip : n_kv - j_lo;
  // key tile visited at position it (0 .. n_tiles-1): descending
  auto tile_of = [&](int it) {
    if constexpr (BSP) {
      const int u = it + bs_skip;
      return 2 * bs_idx[u >> 1] + 1 - (u & 1);
    } else {
      return n_kv - 1 - it;
    }
  };
  float* part_o = SPLIT ? p.part + ((int64_t)split * p.B * p.NH + bh) * T * DV : nullptr;
  float* part_l = SPLIT ? p.part + (int64_t)p.nsplit * p.B * p.NH * T * DV + ((int64_t)split * p.B * p.NH + bh) * T
                        : nullptr;
  if (SPLIT && n_tiles <= 0) {  // an empty key chunk: O = 0, LSE = -inf for the merge
    if (my_q < T) {
#pragma unroll
      for (int y = 0; y < DV / 8; ++y)
        *reinterpret_cast<f32x4*>(part_o + (int64_t)my_q * DV + 8 * y + 4 * g) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (g == 0) part_l[my_q] = -INFINITY;
    }
    return;
  }
  if (q0 >= Lq || n_kv == 0 || (BSP && n_tiles <= 0)) {  // padding rows only, or no keys: O = 0, LSE = -inf
    if (my_q < T) {
      E* orow = og + (int64_t)my_q * p.so.t;
#pragma unroll
      for (int y = 0; y < DV / 8; ++y) *reinterpret_cast<u32x2*>(orow + 8 * y + 4 * g) = u32x2{0u, 0u};
      if (p.lse != nullptr && g == 0) p.lse[(int64_t)bh * T + my_q] = -INFINITY;
    }
    return;
  }

  // Q rows of this wavefront, as B-operand fragments of S^T = K Q^T.
  vec8<E> qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (my_q < Lq) raw = *reinterpret_cast<const u32x4*>(qg + (int64_t)my_q * p.sq.t + 16 * ks + 8 * g);
    qf[ks] = __builtin_bit_cast(vec8<E>, raw);
  }

  DirectTile<FWD_BN, DQK, FWD_NT / 64> kload;
  DirectTile<FWD_BN, DV, FWD_NT / 64> vload;
  kload.init(skt, w, lane);
  vload.init(svt, w, lane);
  auto load_kv = [&](int key0, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    kload.issue(kg + key0 * skt, skt, Lk - key0, (ATTN_LDS char*)(BUF ? kbuf1 : kbuf0), w);
    vload.issue(vg + key0 * svt, svt, Lk - key0, (ATTN_LDS char*)(BUF ? vbuf1 : vbuf0), w);
    if constexpr (KBIAS) {  // this tile's 64 key biases (zero past Lk)
      if (w == 0) load_f32x64_lds(p.kbias + (int64_t)bh * p.kbias_ld + key0, Lk - key0,
                                  (ATTN_LDS float*)(BUF ? kbl1 : kbl0), lane);
    }
  };

  const float c = p.scale_log2;
  // ALiBi in score units: c (s + sl (j - i)) = c s + m_h log2(e) (j - i)
  const float sl = ALIBI ? alibi_slope_log2(h, p.NH) / c : 0.f;

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = zero16();

  load_kv(tile_of(0) * FWD_BN, std::integral_constant<int, 0>{});

  // One key/value tile; BUF is this tile's buffer, the next tile goes to the other one.
  // MASKED: the tile may hold keys past a row's diagonal or past T (the first tiles).
  auto step = [&](int it, auto bufc, auto maskc) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr bool MASKED = decltype(maskc)::value;
    const int j = tile_of(it);  // diagonal / tail tile first
    __builtin_amdgcn_s_waitcnt(0);  // this wave's part of tile j has landed in LDS
    __syncthreads();                // ... and every other wave's; the other buffer is free
    // dropout: this row's keep bits for keys 64 j .. 64 j + 63 (bit k of word k / 32), read
    // before the next tile's loads so that waiting for them leaves those in flight
    u32x2 keepw = {0u, 0u};
    if constexpr (DROP)
      keepw = *reinterpret_cast<const u32x2*>(p.drop_rows + ((int64_t)bh * p.drop_ld * 8 + my_q) * p.drop_ld +
                                              j * (FWD_BN / 8));
    if (it + 1 < n_tiles) load_kv(tile_of(it + 1) * FWD_BN, std::integral_constant<int, 1 - BUF>{});
    const int key0 = j * FWD_BN;
    if (MASKED && CAUSAL && key0 > qw + 31) return;  // tile wholly above this wavefront's rows
    if (MASKED && WIN && key0 + FWD_BN <= qw - W + 1) return;  // wholly below its windows
    const ATTN_LDS char* kt = (const ATTN_LDS char*)(BUF ? kbuf1 : kbuf0);
    const ATTN_LDS char* vt = (const ATTN_LDS char*)(BUF ? vbuf1 : vbuf0);
    // S^T = K Q^T for keys key0 .. key0+63 (two 32-key accumulators)
    f32x16 s0, s1;
    auto scores = [&]() __attribute__((always_inline)) {
      s0 = zero16();
      s1 = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s0 = mfma32(lds_row8<E, FWD_BN>(kt, L, 0, ks), qf[ks], s0);
        s1 = mfma32(lds_row8<E, FWD_BN>(kt, L, 32, ks), qf[ks], s1);
      }
      if constexpr (KBIAS) {  // key of element r: key0 + 8 (r / 4) + 4 g + r % 4 (+32 in s1)
        const float* kb = BUF ? kbl1 : kbl0;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 b0 = *reinterpret_cast<const f32x4*>(kb + 8 * a + 4 * g);
          const f32x4 b1 = *reinterpret_cast<const f32x4*>(kb + 32 + 8 * a + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s0[4 * a + e] += b0[e];
            s1[4 * a + e] += b1[e];
          }
        }
      }
      if constexpr (ALIBI) {  // key of element r: key0 + 8 (r / 4) + 4 g + r % 4 (+32 in s1)
        const float b0 = sl * (float)(key0 + 4 * g - my_q);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] += __builtin_fmaf(sl, (float)(8 * (r >> 2) + (r & 3)), b0);
          s1[r] += __builtin_fmaf(sl, (float)(32 + 8 * (r >> 2) + (r & 3)), b0);
        }
      }
      if constexpr (MASKED) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk0 = key0 + 8 * (r >> 2) + 4 * g + (r & 3), kk1 = kk0 + 32;
          if (kk0 >= Lk || (CAUSAL && (kk0 > my_q || (WIN && my_q - kk0 >= W)))) s0[r] = -INFINITY;
          if (kk1 >= Lk || (CAUSAL && (kk1 > my_q || (WIN && my_q - kk1 >= W)))) s1[r] = -INFINITY;
        }
      }
    };
    // The tile's row maximum (scaled, log2 units).  The IEEE maximum (NaN-propagating)
    // maps onto v_maximum3_f32 with no canonicalising moves of the MFMA results.  The
    // first tile a wave processes holds every one of its rows' own keys, so the running
    // max is finite from then on; a later tile under the window's lower edge may hold no
    // key of a row (its maximum is -inf, which never raises the running max).
    auto tile_max = [&]() __attribute__((always_inline)) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s0[r], s1[r]));
      return max_halves(mx) * c;
    };
    auto raise_max = [&](float m_tile) __attribute__((always_inline)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    };
    // p = 2^(S c - m) as bf16 operands of the second product; returns this lane's sum of
    // the rounded p (the weights O is built from), one v_dot2 with (1, 1) per bf16 pair.
    vec8<E> pb[4];
    auto probs = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = exp2_fast(__builtin_fmaf(s0[r], c, -m_run));
        s1[r] = exp2_fast(__builtin_fmaf(s1[r], c, -m_run));
      }
      pb[0] = pack8<E>(s0, 0);
      pb[1] = pack8<E>(s0, 1);
      pb[2] = pack8<E>(s1, 0);
      pb[3] = pack8<E>(s1, 1);
      return sum_pairs(pb[0], sum_pairs(pb[1], sum_pairs(pb[2], sum_pairs(pb[3], 0.f))));
    };
    scores();
    float rs;
    if constexpr (MASKED) {
      const float m_tile = tile_max();
      // Kept as a branch (the empty volatile asm stops the compiler from turning it into
      // unconditional multiplies): it is taken on a row's first tile and rarely after.
      if (__builtin_expect(__any(m_tile > m_run + kRescaleThreshold), 0)) {
        asm volatile("");
        raise_max(m_tile);
      }
      rs = probs();
    } else {
      // No maximum at all on the common path: p is taken against the running max, and
      // only if some lane's sum exceeds 2^8 (so that a p might) are S recomputed from the
      // K tile still in LDS, the running max raised to the exact one and p redone.  A sum
      // <= 2^8 bounds every p by 2^8, the same bound the masked path keeps.
      rs = probs();
      if (__builtin_expect(__any(rs > kSumLimit), 0)) {
        asm volatile("");
        scores();
        raise_max(tile_max());
        rs = probs();
      }
    }
    l_run += rs;
    if constexpr (DROP) {  // the product takes the kept weights only
#pragma unroll
      for (int m = 0; m < 4; ++m) pb[m] = drop8(pb[m], keep_bits8(m < 2 ? keepw[0] : keepw[1], m & 1, g));
    }
    const vec8<E> pb0 = pb[0], pb1 = pb[1], pb2 = pb[2], pb3 = pb[3];
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      o[dt] = mfma32(lds_col8<E, FWD_BN>(vt, L, 0, 32 * dt), pb0, o[dt]);
      o[dt] = mfma32(lds_col8<E, FWD_BN>(vt, L, 16, 32 * dt), pb1, o[dt]);
      o[dt] = mfma32(lds_col8<E, FWD_BN>(vt, L, 32, 32 * dt), pb2, o[dt]);
      o[dt] = mfma32(lds_col8<E, FWD_BN>(vt, L, 48, 32 * dt), pb3, o[dt]);
    }
  };
  // The first tiles (the workgroup's diagonal ones under the causal mask, or the ragged
  // last key block) carry the mask; the loop over the others has no mask code at all.
  constexpr auto B0 = std::integral_constant<int, 0>{};
  constexpr auto B1 = std::integral_constant<int, 1>{};
  constexpr auto MASK = std::true_type{};
  constexpr auto NOMASK = std::false_type{};
  // Tiles j >= first_masked (visited first) hold keys past Lk or past some row's diagonal;
  // tiles j < j_full (visited last) hold keys below some row's window.
  const int first_ragged = Lk % FWD_BN != 0 ? Lk / FWD_BN : n_kv;
  const int first_masked = min(min(first_ragged, CAUSAL ? q0 / FWD_BN : n_kv), n_kv);
  const int j_full = WIN ? min((max(0, q0 + FWD_BM - W) + FWD_BN - 1) / FWD_BN, first_masked) : 0;
  int n_mask = n_kv - first_masked;
  if constexpr (BSP) {  // the masked tiles are the highest ones, so they lead the list
    n_mask = 0;
    while (n_mask < n_tiles && tile_of(n_mask) >= first_masked) ++n_mask;
  }
  const int mid_end = WIN ? n_tiles - max(0, j_full - j_lo) : n_tiles;
  int it = 0;
  if (qw >= Lq) {
    // Every row of this wavefront is padding (the short last query block of a padded
    // batch, a decode step's single query row, or rows past T): it keeps its share of the
    // workgroup's tile loads and barriers and skips the arithmetic.
    for (; it < n_tiles; ++it) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (it + 1 < n_tiles) {
        if (it & 1)
          load_kv(tile_of(it + 1) * FWD_BN, B0);
        else
          load_kv(tile_of(it + 1) * FWD_BN, B1);
      }
    }
  } else {
    for (; it < n_mask; ++it) {
      if (it & 1)
        step(it, B1, MASK);
      else
        step(it, B0, MASK);
    }
    if ((it & 1) && it < mid_end) step(it++, B1, NOMASK);
    for (; it + 1 < mid_end; it += 2) {
      step(it, B0, NOMASK);
      step(it + 1, B1, NOMASK);
    }
    if (it < mid_end) step(it++, B0, NOMASK);
    if constexpr (WIN) {
      for (; it < n_tiles; ++it) {
        if (it & 1)
          step(it, B1, MASK);
        else
          step(it, B0, MASK);
      }
    }
  }

  // deferred normalisation and stats
  const float l_tot = sum_halves(l_run);
  if constexpr (SPLIT) {  // normalised partial O and LSE of this key chunk, fp32
    if (my_q < T) {
      const bool live = my_q < Lq;
      const float inv = live ? 1.f / l_tot : 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = o[dt][4 * a + e] * inv;
          *reinterpret_cast<f32x4*>(part_o + (int64_t)my_q * DV + 32 * dt + 8 * a + 4 * g) = v;
        }
      if (g == 0) part_l[my_q] = live ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }
  if (my_q < Lq) {
    const float inv = (DROP ? p.drop_scale : 1.f) / l_tot;
    E* orow = og + (int64_t)my_q * p.so.t;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        vec4<E> v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (E)(o[dt][4 * a + e] * inv);
        *reinterpret_cast<vec4<E>*>(orow + 32 * dt + 8 * a + 4 * g) = v;
      }
    if (p.lse != nullptr && g == 0)
      p.lse[(int64_t)bh * T + my_q] = (m_run + log2_fast(l_tot)) * kLn2;
  } else if (my_q < T) {  // padding row of a padded batch: O = 0, LSE = -inf
    E* orow = og + (int64_t)my_q * p.so.t;
#pragma unroll
    for (int y = 0; y < DV / 8; ++y) *reinterpret_cast<u32x2*>(orow + 8 * y + 4 * g) = u32x2{0u, 0u};
    if (p.lse != nullptr && g == 0) p.lse[(int64_t)bh * T + my_q] = -INFINITY;
  }
}

template <class E, int DQK, int DV>
static hipError_t fwd_launch(const FwdParams& p, bool causal, hipStream_t s) {
  const dim3 grid((p.T + FWD_BM - 1) / FWD_BM * p.B * p.NH);
  if (p.drop_rows != nullptr) {
    if (causal)
      hipLaunchKernelGGL((fwd_kernel<E, DQK, DV, true, false, false, false, false, false, true>), grid, dim3(FWD_NT),
                         0, s, p);
    else
      hipLaunchKernelGGL((fwd_kernel<E, DQK, DV, false, false, false, false, false, false, true>), grid,
                         dim3(FWD_NT), 0, s, p);
  } else if (p.kbias != nullptr) {
    if (causal)
      hipLaunchKernelGGL((fwd_kernel<E, DQK, DV, true, false, false, false, false, true>), grid, dim3(FWD_NT), 0, s,
                         p);
    else
      hipLaunchKernelGGL((fwd_kernel<E, DQK, DV, false, false, false, false, false, true>), grid, dim3(FWD_NT), 0,
                         s, p);
  } else if (p.bs.items != nullptr) {
    if (causal)
      hipLaunchKernelGGL((fwd_kernel<E, DQK, DV, true, false, false, false, true>), grid, dim3(FWD_NT), 0, s, p);
    else
      hipLaunchKernelGGL((fwd_kernel<E, DQK, DV, false, false, false, false, true>), grid, dim3(FWD_NT), 0, s, p);
  } else if (!causal)
    hipLaunchKernelGGL((fwd_kernel<E, DQK, DV, false, false, false>), grid, dim3(FWD_NT), 0, s, p);
  else if (p.win < kNoWindow)
    hipLaunchKernelGGL((fwd_kernel<E, DQK, DV, true, true, false>), grid, dim3(FWD_NT), 0, s, p);
  else if (p.alibi)
    hipLaunchKernelGGL((fwd_kernel<E, DQK, DV, true, false, true>), grid, dim3(FWD_NT), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_kernel<E, DQK, DV, true, false, false>), grid, dim3(FWD_NT), 0, s, p);
  return hipGetLastError();
}

template <class E>
static hipError_t fwd_dispatch(const FwdParams& p, int d_qk, int d_v, bool causal, hipStream_t s) {
  if (d_qk == 64 && d_v == 64) return fwd_launch<E, 64, 64>(p, causal, s);
  if (d_qk == 128 && d_v == 128) return fwd_launch<E, 128, 128>(p, causal, s);
  if (d_qk == 192 && d_v == 128) return fwd_launch<E, 192, 128>(p, causal, s);
  return hipErrorInvalidValue;
}

// Merge of the key-split partials: for each query row, O = sum_c e^(LSE_c - LSE) O_c and
// LSE = ln sum_c e^(LSE_c), over the splits in one fixed order.  One thread per row and 8
// columns.
template <class E, int DV>
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdParams p) {
  constexpr int G = DV / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)p.B * p.NH * p.T;
  if (gid >= rows * G) return;
  const int64_t row = gid / G;  // over (b, h, t)
  const int c = (int)(gid % G);
  const int t = (int)(row % p.T);
  const int bh = (int)(row / p.T);
  const int b = bh / p.NH, h = bh % p.NH;
  const int64_t plane = (int64_t)p.B * p.NH * p.T;
  const float* lse_c = p.part + (int64_t)p.nsplit * plane * DV + row;
  float m = -INFINITY;
  for (int k = 0; k < p.nsplit; ++k) m = fmaxf(m, lse_c[k * plane]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
  if (m != -INFINITY) {
    for (int k = 0; k < p.nsplit; ++k) {
      const float wgt = exp2_fast((lse_c[k * plane] - m) * kLog2e);
      const float* oc = p.part + (k * plane + row) * DV + 8 * c;
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(oc), x1 = *reinterpret_cast<const f32x4*>(oc + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += wgt * x0[e];
        acc[4 + e] += wgt * x1[e];
      }
      sum += wgt;
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  vec8<E> v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (E)(acc[e] * inv);
  E* dst = (E*)p.o + b * p.so.b + h * p.so.h + (int64_t)t * p.so.t + 8 * c;
  *reinterpret_cast<u32x4*>(dst) = __builtin_bit_cast(u32x4, v);
  if (p.lse != nullptr && c == 0) p.lse[row] = m == -INFINITY ? -INFINITY : m + log2_fast(sum) * kLn2;
}

template <class E, int DQK, int DV>
static hipError_t fwd_split_t(const FwdParams& p, hipStream_t s) {
  const int nbase = (p.T + FWD_BM - 1) / FWD_BM * p.B * p.NH;
  hipLaunchKernelGGL((fwd_kernel<E, DQK, DV, false, false, false, true>), dim3(nbase * p.nsplit), dim3(FWD_NT), 0,
                     s, p);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const int64_t threads = (int64_t)p.B * p.NH * p.T * (DV / 8);
  hipLaunchKernelGGL((fwd_merge_kernel<E, DV>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <class E>
static hipError_t fwd_split_dispatch(const FwdParams& p, int d_qk, int d_v, hipStream_t s) {
  if (d_qk == 64 && d_v == 64) return fwd_split_t<E, 64, 64>(p, s);
  if (d_qk == 128 && d_v == 128) return fwd_split_t<E, 128, 128>(p, s);
  if (d_qk == 192 && d_v == 128) return fwd_split_t<E, 192, 128>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_split(const FwdParams& p, ElemType et, int d_qk, int d_v, hipStream_t s) {
  return et == ELEM_F16 ? fwd_split_dispatch<f16>(p, d_qk, d_v, s) : fwd_split_dispatch<bf16>(p, d_qk, d_v, s);
}

hipError_t launch_fwd(const FwdParams& p, ElemType et, int d_qk, int d_v, bool causal, hipStream_t s) {
  return et == ELEM_F16 ? fwd_dispatch<f16>(p, d_qk, d_v, causal, s) : fwd_dispatch<bf16>(p, d_qk, d_v, causal, s);
}

}  // namespace attn53
