// Exact attention backward for gfx950.
//
// Pages cited (by title and section):
//   [SA8]  "ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析" 2.1 and A.2 (dV = P^T dO,
//          dP = dO V^T, dS = P * (dP - (dP * P) 1), dQ = dS K / sqrt(d_k), dK = dS^T Q / sqrt(d_k)),
//          4.1 (recompute instead of storing P), 5.3 (simplified softmax-backward term)
//   [2CTA] "深度学习反向传播优化：2-CTA MMA模式与内存访问优化" 2.2 (dQ is a sum over key/value
//          blocks), 3.1 (global atomic accumulation of dQ), 3.2 (deterministic mode,
//          head/batch swizzle, longest-first order), 6.2 (diagonal-first)
//
// Kernels, in stream order:
//   bwd_pre_kernel     D_i = sum_k dO_ik O_ik  (= (dP * P) 1 of [SA8 2.1]: summing
//                      P_ij dP_ij = P_ij sum_k dO_ik V_jk over j gives sum_k dO_ik O_ik)
//                      and LSE_i log2(e) (padding rows +inf), both into the workspace;
//                      clears the fp32 dQ accumulator (atomic mode).
//   bwd_kv_kernel      one workgroup per key/value block of BWD_BN = 128 keys; each of
//                      its 4 wavefronts owns 32 keys, keeps K and V as B operands and dK,
//                      dV as accumulators, and loops over query blocks of BWD_BM = 64:
//                        S = Q K^T, P = 2^(S scale log2e - LSE log2e)  (recomputed)
//                        dP = dO V^T, dS = P * (dP - D)
//                        dV += P^T dO, dK += dS^T Q  (P, dS straight from registers,
//                                                     dO, Q read column-wise from LDS)
//                      atomic mode: dS is staged in LDS, the 64 x d_qk partial dQ = dS K
//                      over this block's keys is formed with MFMAs and added with fp32
//                      atomics into the accumulator [2CTA 3.1].
//   bwd_dq_kernel      deterministic mode only: one workgroup per query block of 128 rows,
//                      looping over key blocks in one fixed order and summing dQ in
//                      registers (S and dP recomputed), so dQ is bit-identical from run
//                      to run; the kv kernel then issues no atomics.
//   bwd_finalize_kernel dQ = scale * accumulator -> bf16 (atomic mode).
#pragma once

#include <type_traits>

#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn53 {

constexpr int BWD_BN = 128;  // keys per workgroup (32 per wavefront)
constexpr int BWD_BM = 64;   // queries per step
constexpr int BWD_NT = 256;
constexpr int DQ_BN = 64;    // dQ kernel: keys per step

// ---------------------------------------------------------------------------------
// preprocess: D = rowsum(dO * O); optional clear of the dQ accumulator
// ---------------------------------------------------------------------------------
// G = DV / 8 lanes per row, 16 bytes of O and of dO each; a workgroup takes NP groups of
// 256 / G rows and issues the loads of all of them before the first sum, so that every
// lane has NP pairs of loads in flight (NP = 4 on large grids, 1 on small ones, which
// need the workgroups more).
template <class E, int DV, int NP>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int d_qk, int zero_acc) {
  constexpr int G = DV / 8;
  constexpr int RPP = 256 / G;  // rows per pass
  const int c = (int)(threadIdx.x % G);
  const int64_t row0 = (int64_t)blockIdx.x * (NP * RPP) + threadIdx.x / G;  // over B * NH * Tpad
  const int64_t nrows = (int64_t)p.B * p.NH * p.Tpad;
  vec8<E> ov[NP], dv[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int64_t row = row0 + (int64_t)k * RPP;
    u32x4 ra = {0u, 0u, 0u, 0u}, rb = {0u, 0u, 0u, 0u};
    if (row < nrows) {
      const int t = (int)(row % p.Tpad);
      const int bh = (int)(row / p.Tpad);
      const int b = bh / p.NH, h = bh % p.NH;
      const int Lq = p.seq_q != nullptr ? batch_len(p.seq_q, b, p.T) : p.T;
      if (t < Lq) {
        const E* orow = (const E*)p.o + b * p.so.b + h * p.so.h + (int64_t)t * p.so.t;
        const E* drow = (const E*)p.dO + b * p.sdo.b + h * p.sdo.h + (int64_t)t * p.sdo.t;
        ra = *reinterpret_cast<const u32x4*>(orow + 8 * c);
        rb = *reinterpret_cast<const u32x4*>(drow + 8 * c);
      }
    }
    ov[k] = __builtin_bit_cast(vec8<E>, ra);
    dv[k] = __builtin_bit_cast(vec8<E>, rb);
  }
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int64_t row = row0 + (int64_t)k * RPP;
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += (float)ov[k][e] * (float)dv[k][e];
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, G);
    if (row < nrows) {
      if (zero_acc) {
        float* acc = p.dq_acc + row * d_qk;
        for (int x = 4 * c; x < d_qk; x += 4 * G) *reinterpret_cast<f32x4*>(acc + x) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (c == 0) {
        const int t = (int)(row % p.Tpad);
        const int bh = (int)(row / p.Tpad);
        p.D[row] = sum;
        // LSE in base-2 units; padding rows (past T, past the batch's query length, or
        // without keys: LSE = -inf) get +inf, which makes their P exactly 0
        const int Lq = p.seq_q != nullptr ? batch_len(p.seq_q, bh / p.NH, p.T) : p.T;
        const float l = t < Lq ? p.lse[(int64_t)bh * p.T + t] : -INFINITY;
        p.lse2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// main backward: key/value-stationary
// ---------------------------------------------------------------------------------
// LDS (d = 128): K block 32 KB (B operand of the partial dQ = dS K), Q and dO tiles
// 2 x 16 KB each (double-buffered direct global->LDS loads), dS^T 2 x 16 KB, LSE and
// D 2 x 256 B each.  Every buffer is its own LDS object so that reads of one buffer
// do not wait for the loads in flight into the other.  Per query block i (one step):
//   top:    wait for this step's tiles, barrier, start the loads of step i+1;
//   dQ:     partial dQ of step i-1 (64 x d_qk) = dS K from the dS^T tile that step
//           left in LDS, then fp32 atomic adds into the accumulator [2CTA 3.1]; the
//           adds drain behind this step's matrix work;
//   S, dP   (2 x d/16 MFMAs each; A operands are row reads of Q / dO);
//   P, dS   on the VALU; dV += P^T dO and dK += dS^T Q with the B operands read
//           column-wise (ds_read_b64_tr_b16);
//   dS^T -> LDS for the next step's dQ.
// With d_qk = 192 LDS holds one dS^T buffer only; a barrier then separates the last
// reads of the previous tile from the writes of the new one.
// Placement of the work of one unmasked step of the key/value kernel, an explicit
// software pipeline for one wavefront.  The step issues N MFMAs in the order
//   S (tile t = 0, then 1; KSQ each), dP (t = 0, then 1; KSV each),
//   dV (P fragment m = 0..3, NDV each), dK (dS fragment m = 0..3, NDK each);
// MFMA i is bundle i.  Every operand read from LDS is issued LA bundles before its
// MFMA.  The VALU work is a list of 72 operations: P elements of tile 0 (with the two
// bf16 packs of that tile after elements 7 and 15), P of tile 1, dS of tile 0, dS of
// tile 1.  They are placed in order, each no earlier than its inputs are ready (two
// bundles after the last MFMA producing them), at most `cap` cost units per bundle
// (P element 6, dS element 3, pack 4; an MFMA bundle lasts 8 VALU issue slots), with
// the smallest cap for which every pack lands before the first MFMA that reads it.
// Rows of LSE and D are read from LDS three bundles before their first use.
template <int DQK, int DV>
struct KvPlan {
  static constexpr int KSQ = DQK / 16, KSV = DV / 16, NDK = DQK / 32, NDV = DV / 32;
  static constexpr int NS = 2 * KSQ, NP = 2 * KSV, NV = 4 * NDV, NK = 4 * NDK;
  static constexpr int N = NS + NP + NV + NK;
  static constexpr int LA = 5, RING = LA + 2;
  static constexpr int NOPS = 72;
  struct Table {
    int bundle[NOPS];
    int lse_bundle[8];
    int d_bundle[8];
    int ok;
  };
  // op o: group o / 18 (0: P tile 0, 1: P tile 1, 2: dS tile 0, 3: dS tile 1);
  // k = o % 18: 0..7 elements 0..7, 8 pack of half 0, 9..16 elements 8..15, 17 pack of half 1
  static constexpr bool is_pack(int o) { return o % 18 == 8 || o % 18 == 17; }
  static constexpr int cost(int o) { return is_pack(o) ? 4 : (o / 18 < 2 ? 6 : 3); }
  static constexpr int earliest(int o) {
    const int grp = o / 18, t = grp & 1;
    return grp < 2 ? KSQ * (t + 1) + 1 : NS + KSV * (t + 1) + 1;
  }
  static constexpr int deadline(int o) {  // packs: the bundle before the first reader
    const int grp = o / 18, t = grp & 1, m = 2 * t + (o % 18 == 8 ? 0 : 1);
    return grp < 2 ? NS + NP + m * NDV - 1 : NS + NP + NV + m * NDK - 1;
  }
  static constexpr Table make(int cap) {
    Table tb{};
    tb.ok = 1;
    int cur = 0, used = 0;
    for (int o = 0; o < NOPS; ++o) {
      if (earliest(o) > cur) {
        cur = earliest(o);
        used = 0;
      }
      if (used > 0 && used + cost(o) > cap) {
        ++cur;
        used = 0;
      }
      tb.bundle[o] = cur;
      used += cost(o);
      if ((is_pack(o) && cur > deadline(o)) || cur >= N) tb.ok = 0;
    }
    for (int x = 0; x < 8; ++x) {
      const int t = x / 4, a = x % 4, k = 4 * a < 8 ? 4 * a : 4 * a + 1;
      const int lb = tb.bundle[t * 18 + k] - 3, db = tb.bundle[(2 + t) * 18 + k] - 3;
      tb.lse_bundle[x] = lb < 0 ? 0 : lb;
      tb.d_bundle[x] = db < 0 ? 0 : db;
    }
    return tb;
  }
  static constexpr Table choose() {
    for (int cap = 6; cap < 64; ++cap)
      if (make(cap).ok) return make(cap);
    return make(64);
  }
  static constexpr Table plan = choose();
  static_assert(plan.ok, "no feasible placement of the step's VALU work");
};

// WIN (with CAUSAL only): sliding window of p.win keys.  ALIBI (with CAUSAL only): the
// linear bias -m_h (i - j) on the scaled scores.  BSP: block-sparse map (p.bs_kv): the
// workgroup visits only the query steps of its key block's live query blocks, ascending.
// KBIAS: a per-key bias (p.kbias) on the scores; each lane's key is fixed, so the bias is
// one register, and the lane sums dS over the queries for dbias (p.dbias_part).
// The body takes its work item's index `bid`: the kernel below passes its workgroup index,
// the merged d = 64 kernel further down a share of its own.
template <class E, int DQK, int DV, bool CAUSAL, bool WIN, bool ALIBI, bool ATOMIC_DQ, bool BSP = false,
          bool KBIAS = false, bool DROP = false>
__device__ __forceinline__ void bwd_kv_body(const BwdParams& p, const int bid) {
  constexpr int KSQ = DQK / 16, KSV = DV / 16;
  constexpr int NDK = DQK / 32, NDV = DV / 32;
  constexpr int NDQ = DQK / 32 / 2;  // dQ tiles per wavefront
  constexpr int QT_BYTES = BWD_BM * DQK * 2;
  constexpr int OT_BYTES = BWD_BM * DV * 2;
  constexpr int KD_BYTES = ATOMIC_DQ ? BWD_BN * DQK * 2 : 16;
  constexpr int ST_BYTES = ATOMIC_DQ ? BWD_BN * BWD_BM * 2 : 16;
  constexpr bool ST_DOUBLE = DQK <= 128;
  __shared__ __attribute__((aligned(1024))) char qbuf0[QT_BYTES], qbuf1[QT_BYTES];
  __shared__ __attribute__((aligned(1024))) char obuf0[OT_BYTES], obuf1[OT_BYTES];
  __shared__ __attribute__((aligned(1024))) char kd_lds[KD_BYTES];
  __shared__ __attribute__((aligned(1024))) char st0[ST_BYTES], st1[ST_DOUBLE ? ST_BYTES : 16];
  __shared__ __attribute__((aligned(256))) float lse0[BWD_BM], lse1[BWD_BM], dd0[BWD_BM], dd1[BWD_BM];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, lq = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: kept in a scalar register
  const int T = p.T;
  // Lq / Lk: valid query / key rows of this batch (T, or the padded-batch lengths)
  int kb, b, h, Lq = T, Lk = T;
  if constexpr (BSP) {  // work list of (b * NH + h, key block), longest first
    const int bhi = p.bs_kv.items[2 * bid];
    kb = p.bs_kv.items[2 * bid + 1];
    b = bhi / p.NH;
    h = bhi % p.NH;
  } else if (p.items_kv == nullptr) {
    const Item item = schedule(bid, p.B * p.NH);
    kb = item.rank;  // causal: block 0 has the most query blocks -> first
    b = item.bh / p.NH;
    h = item.bh % p.NH;
  } else {
    const ListItem it = list_item(bid, p.NH, p.items_kv);
    b = it.b;
    h = it.h;
    kb = it.blk;
    Lq = batch_len(p.seq_q, b, T);
    Lk = batch_len(p.seq_k, b, T);
  }
  const int bh = b * p.NH + h;
  const int nqb = (Lq + BWD_BM - 1) / BWD_BM;

  const E* qg = (const E*)p.q + b * p.sq.b + h * p.sq.h;
  const E* kg = (const E*)p.k + b * p.sk.b + h * p.sk.h;
  const E* vg = (const E*)p.v + b * p.sv.b + h * p.sv.h;
  const E* dog = (const E*)p.dO + b * p.sdo.b + h * p.sdo.h;
  const float* lseg = p.lse2 + (int64_t)bh * p.Tpad;
  const float* Dg = p.D + (int64_t)bh * p.Tpad;
  const int64_t sqt = p.sq.t, sdot = p.sdo.t;

  const LdsLane L = lds_lane(lane);
  const int key0 = kb * BWD_BN;
  const int kw = 32 * w;
  const int my_key = key0 + kw + lq;
  const float c = p.scale_log2;
  const float ml = ALIBI ? alibi_slope_log2(h, p.NH) : 0.f;  // ALiBi slope, log2 units
  // key bias of this lane's key in log2 units, and this lane's partial sums of dS
  const float kb2 = KBIAS ? p.kbias[(int64_t)bh * p.Tpad + min(my_key, p.Tpad - 1)] * c : 0.f;
  float dbacc[2] = {0.f, 0.f};
  E* dkg = (E*)p.dk + b * p.sdk.b + h * p.sdk.h;
  E* dvg = (E*)p.dv + b * p.sdv.b + h * p.sdv.h;

  const int W = WIN ? p.win : kNoWindow;
  const int i0 = CAUSAL ? key0 / BWD_BM : 0;
  // sliding window: query blocks past i_end hold no query whose window reaches this block
  const int i_end = WIN ? min(nqb, (key0 + BWD_BN - 1 + W - 1) / BWD_BM + 1) : nqb;
  // Block-sparse: the live query blocks (ascending) hold two steps of 64 rows each; the
  // upper step of the last one may lie wholly past Lq and is then left out.
  const int* bs_idx = BSP ? p.bs_kv.idx + ((int64_t)bh * p.bs_kv.nb + kb) * p.bs_kv.nb : nullptr;
  const int bs_cnt = BSP ? p.bs_kv.cnt[bh * p.bs_kv.nb + kb] : 0;
  const int bs_skip = (BSP && bs_cnt > 0 && bs_idx[bs_cnt - 1] * kBsBlock + BWD_BM >= Lq) ? 1 : 0;
  const int n_q = BSP ? 2 * bs_cnt - bs_skip : i_end - i0;
  // query step (64 rows) visited at position it
  auto qstep = [&](int it) {
    if constexpr (BSP)
      return 2 * bs_idx[it >> 1] + (it & 1);
    else
      return i0 + it;
  };
  if (key0 >= Lk || n_q <= 0) {  // padding keys only, or no query sees them: dK = dV = 0
    if (my_key < T) {
#pragma unroll
      for (int x = 0; x < DQK / 16; ++x)
        *reinterpret_cast<u32x4*>(dkg + (int64_t)my_key * p.sdk.t + g * (DQK / 2) + 8 * x) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int x = 0; x < DV / 16; ++x)
        *reinterpret_cast<u32x4*>(dvg + (int64_t)my_key * p.sdv.t + g * (DV / 2) + 8 * x) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }

  // K and V rows of this wavefront as B-operand fragments of S = Q K^T and dP = dO V^T.
  vec8<E> kf[KSQ], vf[KSV];
#pragma unroll
  for (int ks = 0; ks < KSQ; ++ks) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (my_key < Lk) raw = *reinterpret_cast<const u32x4*>(kg + (int64_t)my_key * p.sk.t + 16 * ks + 8 * g);
    kf[ks] = __builtin_bit_cast(vec8<E>, raw);
  }
#pragma unroll
  for (int ks = 0; ks < KSV; ++ks) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (my_key < Lk) raw = *reinterpret_cast<const u32x4*>(vg + (int64_t)my_key * p.sv.t + 16 * ks + 8 * g);
    vf[ks] = __builtin_bit_cast(vec8<E>, raw);
  }

  DirectTile<BWD_BM, DQK, BWD_NT / 64> qload;
  DirectTile<BWD_BM, DV, BWD_NT / 64> oload;
  qload.init(sqt, w, lane);
  oload.init(sdot, w, lane);
  auto load_step = [&](int qb, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int r0 = qb * BWD_BM;
    qload.issue(qg + r0 * sqt, sqt, Lq - r0, (ATTN_LDS char*)(BUF ? qbuf1 : qbuf0), w);
    oload.issue(dog + r0 * sdot, sdot, Lq - r0, (ATTN_LDS char*)(BUF ? obuf1 : obuf0), w);
    if (w == 0) {  // 64 rows of LSE log2(e) and of D (both padded to Tpad rows)
      load_f32x64_lds(lseg + r0, BWD_BM, (ATTN_LDS float*)(BUF ? lse1 : lse0), lane);
    } else if (w == 1) {
      load_f32x64_lds(Dg + r0, BWD_BM, (ATTN_LDS float*)(BUF ? dd1 : dd0), lane);
    }
  };

  if constexpr (ATOMIC_DQ) {
    TileStage<BWD_BN, DQK, BWD_NT> kst;
    kst.load(kg, p.sk.t, key0, Lk, tid);
    kst.store((ATTN_LDS char*)kd_lds, tid);
  }


  f32x16 dk[NDK], dv[NDV];
#pragma unroll
  for (int t = 0; t < NDK; ++t) dk[t] = zero16();
#pragma unroll
  for (int t = 0; t < NDV; ++t) dv[t] = zero16();
  const int tq = w & 1;               // dQ: query tile of this wavefront
  const int dq_t0 = (w >> 1) * NDQ;   //     first d tile
  float* dqacc = ATOMIC_DQ ? p.dq_acc + (int64_t)bh * p.Tpad * DQK : nullptr;

  // partial dQ of the query block at q0 from the dS^T tile in `st`, added atomically
  auto dq_partial = [&](const ATTN_LDS char* st, int q0) {
    f32x16 dq[NDQ];
#pragma unroll
    for (int n = 0; n < NDQ; ++n) dq[n] = zero16();
    const ATTN_LDS char* kd = (const ATTN_LDS char*)kd_lds;
#pragma unroll
    for (int m = 0; m < BWD_BN / 16; ++m) {
      const vec8<E> a = lds_col8<E, BWD_BN>(st, L, 16 * m, 32 * tq);
#pragma unroll
      for (int n = 0; n < NDQ; ++n) dq[n] = mfma32(a, lds_col8<E, BWD_BN>(kd, L, 16 * m, 32 * (dq_t0 + n)), dq[n]);
    }
#pragma unroll
    for (int n = 0; n < NDQ; ++n) {
      const int d = 32 * (dq_t0 + n) + lq;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + 32 * tq + 8 * (r >> 2) + 4 * g + (r & 3);  // < Tpad
        unsafeAtomicAdd(dqacc + (int64_t)q * DQK + d, dq[n][r]);
      }
    }
  };

  load_step(qstep(0), std::integral_constant<int, 0>{});

  // One query block.  MASKED: the block touches the diagonal or a ragged edge.  The
  // body is one basic block in source order S, dP, P, dV, dS, dK so that the matrix
  // work of dP and dV can run beside the VALU work of P and dS.  keepc (dropout): this
  // lane's key's keep bits for the block's 64 queries (bit k of word k / 32).
  auto step_body = [&](int q0, auto bufc, auto maskc, const u32x2& keepc) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr bool MASKED = decltype(maskc)::value;
    ATTN_LDS char* st_cur = (ATTN_LDS char*)((ST_DOUBLE && BUF) ? st1 : st0);
    const ATTN_LDS char* qt = (const ATTN_LDS char*)(BUF ? qbuf1 : qbuf0);
    const ATTN_LDS char* ot = (const ATTN_LDS char*)(BUF ? obuf1 : obuf0);
    const float* lb = BUF ? lse1 : lse0;
    const float* db = BUF ? dd1 : dd0;
    // ALiBi: m_h log2(e) (key - query) = ab - ml (32 t + 8 (r / 4) + r % 4) for element r of
    // tile t (query q0 + 32 t + 8 (r / 4) + 4 g + r % 4, key my_key)
    const float ab = ALIBI ? ml * (float)(my_key - q0 - 4 * g) : 0.f;
    if (MASKED && CAUSAL && (key0 + kw > q0 + BWD_BM - 1 || (WIN && q0 - (key0 + kw + 31) >= W))) {
      // every key of this wavefront lies above every query of the block, or below every
      // query's window: P = dS = 0
      if constexpr (ATOMIC_DQ) {
        if constexpr (!ST_DOUBLE) __syncthreads();
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          *reinterpret_cast<ATTN_LDS u32x2*>(st_cur + tile_off<BWD_BN>(kw + lq, 16 * m + 4 * g)) = u32x2{0u, 0u};
          *reinterpret_cast<ATTN_LDS u32x2*>(st_cur + tile_off<BWD_BN>(kw + lq, 16 * m + 8 + 4 * g)) = u32x2{0u, 0u};
        }
      }
      return;
    }
    f32x16 s[2], dp[2];
    vec8<E> pb[4], sb[4];
    // MASKED: P = 0 for this lane's key past Lk, a query past Lq, the key past the query's
    // diagonal or under its window; element r of tile t is query q0 + 32 t + 8 (r / 4) +
    // 4 g + r % 4, so query - key = qk + 32 t + 8 (r / 4) + r % 4 and Lq - query =
    // lqr - (32 t + 8 (r / 4) + r % 4)
    const int qk = q0 + 4 * g - my_key, lqr = Lq - q0 - 4 * g;
    const bool key_ok = my_key < Lk;
    // d_qk = 128 runs its masked steps in the pipeline too; at d_qk = 64 (two wavefronts
    // per SIMD, 256 registers) and 192 the pipeline's masked form spills, so their masked
    // steps keep the plain, compiler-scheduled body
    if constexpr (MASKED && DQK != 128) {
      // S = Q K^T and dP = dO V^T for 64 queries x this wavefront's 32 keys
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          s[t] = mfma32(lds_row8<E, BWD_BM>(qt, L, 32 * t, ks), kf[ks], ks == 0 ? zero16() : s[t]);
#pragma unroll
      for (int ks = 0; ks < KSV; ++ks)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          dp[t] = mfma32(lds_row8<E, BWD_BM>(ot, L, 32 * t, ks), vf[ks], ks == 0 ? zero16() : dp[t]);
      // P = 2^(S c - LSE log2 e); element r of tile t: query q0 + 32 t + 8 (r / 4) + 4 g + r % 4
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int qi = 32 * t + 8 * a + 4 * g;
          const f32x4 Lv = *reinterpret_cast<const f32x4*>(lb + qi);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * a + e;
            const int q = q0 + qi + e;
            const float bias = (ALIBI ? __builtin_fmaf(-ml, (float)(32 * t + 8 * a + e), ab) : 0.f) + kb2;
            const float pv = exp2_fast(__builtin_fmaf(s[t][r], c, bias - Lv[e]));
            s[t][r] = (my_key >= Lk || q >= Lq || (CAUSAL && (my_key > q || (WIN && q - my_key >= W)))) ? 0.f : pv;
          }
        }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        pb[m] = pack8<E>(s[m >> 1], m & 1);
        if constexpr (DROP) pb[m] = drop8(pb[m], keep_bits8(keepc[m >> 1], m & 1, g));
      }
      // dV += P^T dO  (contraction over the 64 queries)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < NDV; ++t) dv[t] = mfma32(pb[m], lds_col8<E, BWD_BM>(ot, L, 16 * m, 32 * t), dv[t]);
      // dS = P (dP - D)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 Dd = *reinterpret_cast<const f32x4*>(db + 32 * t + 8 * a + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float dpk = dp[t][4 * a + e];
            if constexpr (DROP) dpk = ((keepc[t] >> (8 * a + 4 * g + e)) & 1u) ? dpk * p.drop_scale : 0.f;
            dp[t][4 * a + e] = s[t][4 * a + e] * (dpk - Dd[e]);
            if constexpr (KBIAS) dbacc[t] += dp[t][4 * a + e];
          }
        }
#pragma unroll
      for (int m = 0; m < 4; ++m) sb[m] = pack8<E>(dp[m >> 1], m & 1);
      // dK += dS^T Q
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < NDK; ++t) dk[t] = mfma32(sb[m], lds_col8<E, BWD_BM>(qt, L, 16 * m, 32 * t), dk[t]);
    } else {
      // An explicit pipeline (KvPlan): bundle i issues MFMA i, the
      // operand read of MFMA i + LA and its share of the VALU work; the compiler may
      // reorder only within a bundle.
      using Plan = KvPlan<DQK, DV>;
      constexpr int NS = Plan::NS, NP = Plan::NP, NV = Plan::NV, LA = Plan::LA, RING = Plan::RING;
      vec8<E> fr[RING];
      f32x4 lsev[2][4], ddv[2][4];
      f32x16 pv[2], dsv[2];  // P and dS, apart from the S and dP accumulators
      auto read_frag = [&](auto jc) -> vec8<E> {
        constexpr int j = decltype(jc)::value;
        if constexpr (j < NS) {
          return lds_row8<E, BWD_BM>(qt, L, 32 * (j / KSQ), j % KSQ);
        } else if constexpr (j < NS + NP) {
          return lds_row8<E, BWD_BM>(ot, L, 32 * ((j - NS) / KSV), (j - NS) % KSV);
        } else if constexpr (j < NS + NP + NV) {
          return lds_col8<E, BWD_BM>(ot, L, 16 * ((j - NS - NP) / NDV), 32 * ((j - NS - NP) % NDV));
        } else {
          return lds_col8<E, BWD_BM>(qt, L, 16 * ((j - NS - NP - NV) / NDK), 32 * ((j - NS - NP - NV) % NDK));
        }
      };
      auto valu_op = [&](auto oc) {
        constexpr int o = decltype(oc)::value;
        constexpr int grp = o / 18, k = o % 18, t = grp & 1;
        constexpr int h = k < 9 ? 0 : 1, r = k < 8 ? k : k - 1;
        if constexpr (grp < 2) {
          if constexpr (Plan::is_pack(o)) {
            pb[2 * t + h] = pack8<E>(pv[t], h);
            if constexpr (DROP) pb[2 * t + h] = drop8(pb[2 * t + h], keep_bits8(keepc[t], h, g));
          } else
          {
            if constexpr (ALIBI) {
              const float bias = __builtin_fmaf(-ml, (float)(32 * t + 8 * (r >> 2) + (r & 3)), ab);
              pv[t][r] = exp2_fast(__builtin_fmaf(s[t][r], c, bias - lsev[t][r >> 2][r & 3]));
            } else if constexpr (KBIAS) {
              pv[t][r] = exp2_fast(__builtin_fmaf(s[t][r], c, kb2 - lsev[t][r >> 2][r & 3]));
            } else {
              pv[t][r] = exp2_fast(__builtin_fmaf(s[t][r], c, -lsev[t][r >> 2][r & 3]));
            }
            if constexpr (MASKED) {
              constexpr int off = 32 * t + 8 * (r >> 2) + (r & 3);
              const int d = qk + off;  // query - key
              pv[t][r] = (!key_ok || off >= lqr || (CAUSAL && (d < 0 || (WIN && d >= W)))) ? 0.f : pv[t][r];
            }
          }
        } else {
          if constexpr (Plan::is_pack(o))
            sb[2 * t + h] = pack8<E>(dsv[t], h);
          else {
            float dpk = dp[t][r];
            if constexpr (DROP) dpk = ((keepc[t] >> (8 * (r >> 2) + 4 * g + (r & 3))) & 1u) ? dpk * p.drop_scale : 0.f;
            dsv[t][r] = pv[t][r] * (dpk - ddv[t][r >> 2][r & 3]);
            if constexpr (KBIAS) dbacc[t] += dsv[t][r];
          }
        }
      };
      static_for<0, LA>([&](auto jc) { fr[decltype(jc)::value % RING] = read_frag(jc); });
      ATTN_SCHED_FENCE();
      static_for<0, Plan::N>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const vec8<E> f = fr[i % RING];
        if constexpr (i < NS) {
          constexpr int t = i / KSQ, ks = i % KSQ;
          s[t] = mfma32(f, kf[ks], ks == 0 ? zero16() : s[t]);
        } else if constexpr (i < NS + NP) {
          constexpr int t = (i - NS) / KSV, ks = (i - NS) % KSV;
          dp[t] = mfma32(f, vf[ks], ks == 0 ? zero16() : dp[t]);
        } else if constexpr (i < NS + NP + NV) {
          constexpr int m = (i - NS - NP) / NDV, n = (i - NS - NP) % NDV;
          dv[n] = mfma32(pb[m], f, dv[n]);
        } else {
          constexpr int m = (i - NS - NP - NV) / NDK, n = (i - NS - NP - NV) % NDK;
          dk[n] = mfma32(sb[m], f, dk[n]);
        }
        if constexpr (i + LA < Plan::N) fr[(i + LA) % RING] = read_frag(std::integral_constant<int, i + LA>{});
        static_for<0, 8>([&](auto xc) {
          constexpr int x = decltype(xc)::value, t = x / 4, a = x % 4;
          if constexpr (Plan::plan.lse_bundle[x] == i)
            lsev[t][a] = *reinterpret_cast<const f32x4*>(lb + 32 * t + 8 * a + 4 * g);
          if constexpr (Plan::plan.d_bundle[x] == i)
            ddv[t][a] = *reinterpret_cast<const f32x4*>(db + 32 * t + 8 * a + 4 * g);
        });
        static_for<0, Plan::NOPS>([&](auto oc) {
          if constexpr (Plan::plan.bundle[decltype(oc)::value] == i) valu_op(oc);
        });
        ATTN_SCHED_FENCE();
      });
    }
    if constexpr (ATOMIC_DQ) {
      if constexpr (!ST_DOUBLE) __syncthreads();  // every wave has read the previous dS^T
      // dS^T tile in LDS: row = key (128), column = query (64); sb[m] holds queries
      // 16 m + 4 g + {0..3} (elements 0..3) and 16 m + 8 + 4 g + {0..3} (elements 4..7)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const u32x4 v = __builtin_bit_cast(u32x4, sb[m]);
        *reinterpret_cast<ATTN_LDS u32x2*>(st_cur + tile_off<BWD_BN>(kw + lq, 16 * m + 4 * g)) = u32x2{v[0], v[1]};
        *reinterpret_cast<ATTN_LDS u32x2*>(st_cur + tile_off<BWD_BN>(kw + lq, 16 * m + 8 + 4 * g)) = u32x2{v[2], v[3]};
      }
    }
  };

  auto step = [&](int it, auto bufc, auto maskc) {
    constexpr int BUF = decltype(bufc)::value;
    const int qb = qstep(it);
    const int q0 = qb * BWD_BM;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads (and its atomics of the step before) are done
    __syncthreads();                // every wave's tiles are in; the other buffers are free
    // dropout keep bits of this lane's key for the block's 64 queries, read before the next
    // step's loads so that waiting for them leaves those in flight
    u32x2 keepc = {0u, 0u};
    if constexpr (DROP)
      keepc = *reinterpret_cast<const u32x2*>(p.drop_cols + ((int64_t)bh * p.drop_tp + my_key) * p.drop_ld + q0 / 8);
    if (it + 1 < n_q) load_step(qstep(it + 1), std::integral_constant<int, 1 - BUF>{});
    if constexpr (ATOMIC_DQ) {
      if (it > 0) dq_partial((const ATTN_LDS char*)((ST_DOUBLE && !BUF) ? st1 : st0), qstep(it - 1) * BWD_BM);
    }
    step_body(q0, bufc, maskc, keepc);
  };
  // The steps that touch the diagonal (the first BWD_BN / BWD_BM under the causal mask),
  // a ragged key block (all steps) or the ragged last query block carry the mask; they
  // are peeled off the loop (their pipeline or plain body applies the mask) so that the
  // loop's body is one straight-line program without mask code.
  constexpr auto MASK = std::true_type{};
  constexpr auto NOMASK = std::false_type{};
  constexpr auto B0 = std::integral_constant<int, 0>{};
  constexpr auto B1 = std::integral_constant<int, 1>{};
  const bool ragged_keys = key0 + BWD_BN > Lk;
  // block-sparse: only a live diagonal block (the first in the list) carries the causal mask
  const bool diag_first = !BSP || (bs_cnt > 0 && bs_idx[0] == kb);
  const int n_head = ragged_keys ? n_q : ((CAUSAL && diag_first) ? min(BWD_BN / BWD_BM, n_q) : 0);  // even, or n_q
  const int n_tail = (n_head < n_q && qstep(n_q - 1) * BWD_BM + BWD_BM > Lq) ? 1 : 0;
  // sliding window: steps from win_start on hold a query past the window of key0
  const int x_win = key0 + W - BWD_BM + 1;
  const int win_start = WIN ? max(n_head, (x_win <= 0 ? 0 : (x_win + BWD_BM - 1) / BWD_BM) - i0) : n_q;
  const int mid_end = WIN ? min(n_q - n_tail, win_start) : n_q - n_tail;
  for (int it = 0; it < n_head; it += 2) {
    step(it, B0, MASK);
    if (it + 1 < n_head) step(it + 1, B1, MASK);
  }
  int it = n_head;
  for (; it + 1 < mid_end; it += 2) {
    step(it, B0, NOMASK);
    step(it + 1, B1, NOMASK);
  }
  if (it < mid_end) step(it++, B0, NOMASK);
  if constexpr (WIN) {
    for (; it < n_q; ++it) {
      if (it & 1)
        step(it, B1, MASK);
      else
        step(it, B0, MASK);
    }
  } else if (it < n_q) {
    if (it & 1)
      step(it, B1, MASK);
    else
      step(it, B0, MASK);
  }
  if constexpr (ATOMIC_DQ) {
    __syncthreads();  // the last dS^T tile is complete
    const bool last_odd = ((n_q - 1) & 1) != 0;
    dq_partial((const ATTN_LDS char*)((ST_DOUBLE && last_odd) ? st1 : st0), qstep(n_q - 1) * BWD_BM);
  }

  if constexpr (KBIAS) {  // dbias_j = sum over queries of dS_ij: this lane's two halves
    const float tot = sum_halves(dbacc[0] + dbacc[1]);
    if (p.dbias_part != nullptr && g == 0 && my_key < T) p.dbias_part[(int64_t)bh * p.Tpad + my_key] = tot;
  }
  // dK = scale dS^T Q, dV; element r of tile t: key key0 + kw + 8 (r / 4) + 4 g + r % 4,
  // column 32 t + lq.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = key0 + kw + 8 * (r >> 2) + 4 * g + (r & 3);
    if (key < T) {
#pragma unroll
      for (int t = 0; t < NDK; ++t) dkg[(int64_t)key * p.sdk.t + 32 * t + lq] = (E)(dk[t][r] * p.scale);
#pragma unroll
      for (int t = 0; t < NDV; ++t) dvg[(int64_t)key * p.sdv.t + 32 * t + lq] = (E)(DROP ? dv[t][r] * p.drop_scale : dv[t][r]);
    }
  }
}

template <class E, int DQK, int DV, bool CAUSAL, bool WIN, bool ALIBI, bool ATOMIC_DQ, bool BSP = false,
          bool KBIAS = false, bool DROP = false>
__global__ __launch_bounds__(BWD_NT) __attribute__((amdgpu_waves_per_eu(DQK == 64 ? 2 : 1, DQK == 64 ? 2 : 1))) void bwd_kv_kernel(BwdParams p) {
  bwd_kv_body<E, DQK, DV, CAUSAL, WIN, ALIBI, ATOMIC_DQ, BSP, KBIAS, DROP>(p, (int)blockIdx.x);
}

// ---------------------------------------------------------------------------------
// dQ without atomics: query-stationary, fixed key-block order
// ---------------------------------------------------------------------------------
// One workgroup of 4 wavefronts per DQ_QT * 128 query rows; each wavefront owns
// DQ_QT tiles of 32 rows, held in registers as B operands together with their dO rows,
// LSE and D.  With two tiles per wavefront (d_qk = 128; one wavefront per SIMD) every
// K or V fragment read from LDS feeds two products; with d_qk = 192 a wavefront owns
// one tile (two do not fit in 512 registers); with d_qk = 64 a wavefront owns one tile
// and two wavefronts share a SIMD (short sequences: twice the workgroups, half the
// work per workgroup).  Key/value tiles of 64 rows stream through
// double-buffered LDS by direct loads, in descending order.  Per tile:
// S^T = K Q^T and dP^T = V dO^T, P^T = 2^(S^T c - LSE log2 e), dS^T = P^T (dP^T - D),
// dQ^T += K^T dS^T with the K^T operand read column-wise.  Every dQ row is summed over
// the key blocks in one fixed order inside one wavefront, so the result is
// bit-identical from run to run.
// Placement of the work of one unmasked key tile in the dQ kernel (explicit pipeline).
// Bundle b issues one LDS operand read (for bundle b + LA) and the QT MFMAs that share
// the fragment of bundle b, in the order S (key half t = 0), dP (t = 0), S (t = 1),
// dP (t = 1), dQ over t = 0, dQ over t = 1.  The VALU work: P of half 0 (QT x 16
// elements), dS of half 0 with the bf16 pack of each group of eight, then the same for
// half 1; placed greedily (P element 6, dS element 3, pack 4 cost units) no earlier
// than two bundles after the MFMAs producing its inputs, with the smallest per-bundle
// budget for which every pack lands before the dQ bundles that read it.
template <int DQK, int DV, int QT, bool KBIAS = false, bool DROP = false>
struct DqPlan {
  static constexpr int KSQ = DQK / 16, KSV = DV / 16, NDQ = DQK / 32;
  static constexpr int S0 = 0, P0 = KSQ, S1 = KSQ + KSV, P1 = 2 * KSQ + KSV, Q0 = 2 * KSQ + 2 * KSV;
  static constexpr int Q1 = Q0 + 2 * NDQ, N = Q1 + 2 * NDQ;
  static constexpr int LA = 4, RING = LA + 1;
  static constexpr int PER = 16 * QT + 2 * QT;  // ops per half: P elements, then dS elements + packs
  static constexpr int NOPS = 2 * (16 * QT + 18 * QT);
  // op o: half t = o / (34 QT); within: k < 16 QT: P element (u = k / 16, r = k % 16);
  // else k' = k - 16 QT: u = k' / 18, e = k' % 18: e = 8 pack half 0, e = 17 pack half 1,
  // else dS element r = e < 8 ? e : e - 1.
  static constexpr int half(int o) { return o / (34 * QT); }
  static constexpr bool is_p(int o) { return o % (34 * QT) < 16 * QT; }
  static constexpr bool is_pack(int o) {
    return !is_p(o) && ((o % (34 * QT) - 16 * QT) % 18 == 8 || (o % (34 * QT) - 16 * QT) % 18 == 17);
  }
  // a key bias adds one FMA to a P element; dropout a bit extract and a mask (the dP
  // multiplier, 1 / (1 - p) or 0) to a dS element, whose subtraction becomes an FMA
  static constexpr int cost(int o) { return is_p(o) ? (KBIAS ? 7 : 6) : (is_pack(o) ? 4 : (DROP ? 5 : 3)); }
  static constexpr int earliest(int o) {
    const int t = half(o);
    return is_p(o) ? (t ? P1 : P0) + 1 : (t ? Q0 : S1) + 1;
  }
  static constexpr int deadline(int o) { return (half(o) ? Q1 : Q0) - 1; }
  struct Table {
    int bundle[NOPS];
    int kb_bundle[2];  // key bias: the bundle that reads half t's 32 bias values from LDS
    int ok;
  };
  static constexpr Table make(int cap) {
    Table tb{};
    tb.ok = 1;
    int cur = 0, used = 0;
    for (int o = 0; o < NOPS; ++o) {
      if (earliest(o) > cur) {
        cur = earliest(o);
        used = 0;
      }
      if (used > 0 && used + cost(o) > cap) {
        ++cur;
        used = 0;
      }
      tb.bundle[o] = cur;
      used += cost(o);
      if ((is_pack(o) && cur > deadline(o)) || cur >= N) tb.ok = 0;
    }
    // two bundles before the half's first P element, and after the other half's last
    const int first0 = tb.bundle[0], first1 = tb.bundle[34 * QT], last0 = tb.bundle[16 * QT - 1];
    tb.kb_bundle[0] = first0 >= 2 ? first0 - 2 : 0;
    tb.kb_bundle[1] = first1 - 2 > last0 ? first1 - 2 : last0 + 1;
    if (tb.kb_bundle[1] > first1) tb.ok = 0;
    return tb;
  }
  static constexpr Table choose() {
    for (int cap = 8; cap < 256; ++cap)
      if (make(cap).ok) return make(cap);
    return make(256);
  }
  static constexpr Table plan = choose();
  static_assert(plan.ok, "no feasible placement of the tile's VALU work");
};

template <int DQK>
struct DqShape {
  static constexpr int QT = DQK == 128 ? 2 : 1;  // 32-row query tiles per wavefront
  static constexpr int BM = 128 * QT;            // query rows per workgroup
  // d_qk = 128, 192: one wavefront per SIMD (up to 512 registers; with d_qk = 192 and
  // one tile, two wavefronts per SIMD of 256 registers each spill about 370 registers per
  // lane); d_qk = 64 with one tile fits 256 registers, so two wavefronts share a SIMD
  static constexpr int WAVES_PER_EU = DQK == 64 ? 2 : 1;
};

// WIN (with CAUSAL only): sliding window of p.win keys.  ALIBI (with CAUSAL only): the
// linear bias -m_h (i - j) on the scaled scores.  BSP: block-sparse map (p.bs_dq): the
// workgroup visits the key tiles of the live key blocks of any of its query-block rows,
// descending; a wavefront computes only on the tiles live for its own rows.  KBIAS: a
// per-key bias (p.kbias) on the scores, 64 values per key tile in LDS, read into
// registers half a tile at a time inside the pipeline.  DROP: dropout keep bits
// (p.drop_rows), one 64-bit word per row and key tile, applied to dP.
template <class E, int DQK, int DV, bool CAUSAL, bool WIN, bool ALIBI, bool BSP = false, bool KBIAS = false,
          bool DROP = false>
__device__ __forceinline__ void bwd_dq_body(const BwdParams& p, const int bid) {
  constexpr int KSQ = DQK / 16, KSV = DV / 16, NDQ = DQK / 32;
  constexpr int QT = DqShape<DQK>::QT, BM = DqShape<DQK>::BM;
  constexpr int KT_BYTES = DQ_BN * DQK * 2;
  constexpr int VT_BYTES = DQ_BN * DV * 2;
  __shared__ __attribute__((aligned(1024))) char kbuf0[KT_BYTES], kbuf1[KT_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[VT_BYTES], vbuf1[VT_BYTES];
  __shared__ __attribute__((aligned(256))) float kbl0[KBIAS ? DQ_BN : 1], kbl1[KBIAS ? DQ_BN : 1];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, lq = lane & 31;
  const int w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the same, in a scalar register
  const int T = p.T;
  const int nqb = (T + BM - 1) / BM;
  // Lq / Lk: valid query / key rows of this batch (T, or the padded-batch lengths)
  int qb, b, h, Lq = T, Lk = T;
  if constexpr (BSP) {  // work list of (b * NH + h, query block of BM rows), longest first
    const int bhi = p.bs_dq.items[2 * bid];
    qb = p.bs_dq.items[2 * bid + 1];
    b = bhi / p.NH;
    h = bhi % p.NH;
  } else if (p.items_dq == nullptr) {
    const Item item = schedule(bid, p.B * p.NH);
    qb = CAUSAL ? nqb - 1 - item.rank : item.rank;
    b = item.bh / p.NH;
    h = item.bh % p.NH;
  } else {
    const ListItem it = list_item(bid, p.NH, p.items_dq);
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
  const E* dog = (const E*)p.dO + b * p.sdo.b + h * p.sdo.h;
  E* dqg = (E*)p.dq + b * p.sdq.b + h * p.sdq.h;
  const int64_t skt = p.sk.t, svt = p.sv.t;

  const LdsLane L = lds_lane(lane);
  const int q0 = qb * BM, qw = q0 + 32 * QT * w;  // first row of this wavefront
  const float c = p.scale_log2;
  const float ml = ALIBI ? alibi_slope_log2(h, p.NH) : 0.f;  // ALiBi slope, log2 units
  const int W = WIN ? p.win : kNoWindow;
  const int kv_end = CAUSAL ? min(Lk, q0 + BM) : Lk;
  const int n_kv = (kv_end + DQ_BN - 1) / DQ_BN;
  // sliding window: tiles below j_lo hold no key of any row's window
  const int j_lo = WIN ? max(0, q0 - W + 1) / DQ_BN : 0;
  // Block-sparse: the live key blocks of the workgroup's query-block rows (descending, with
  // a bit per row) hold two tiles each; the upper tile of the highest one may lie wholly
  // past kv_end and is then left out.  Row bit of this wavefront: its 128-row block.
  const int* bs_idx = BSP ? p.bs_dq.idx + ((int64_t)bh * nqb + qb) * p.bs_dq.nb : nullptr;
  const int bs_cnt = BSP ? p.bs_dq.cnt[bh * nqb + qb] : 0;
  const int bs_skip = (BSP && bs_cnt > 0 && (bs_idx[0] & 0xffff) * kBsBlock + DQ_BN >= kv_end) ? 1 : 0;
  const int bs_row = 16 + (32 * QT * wu) / kBsBlock;
  const int n_tiles = BSP ? 2 * bs_cnt - bs_skip : n_kv - j_lo;
  if (q0 >= Lq || n_kv == 0 || (BSP && n_tiles <= 0)) {  // padding rows only, or no keys: dQ = 0
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      const int q = qw + 32 * u + lq;
      if (q < T) {
#pragma unroll
        for (int x = 0; x < DQK / 16; ++x)
          *reinterpret_cast<u32x4*>(dqg + (int64_t)q * p.sdq.t + g * (DQK / 2) + 8 * x) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    return;
  }

  // Q and dO rows as B operands of S^T = K Q^T and dP^T = V dO^T
  vec8<E> qf[QT][KSQ], df[QT][KSV];
  float lse2[QT], Dq[QT];
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int q = qw + 32 * u + lq;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (q < Lq) raw = *reinterpret_cast<const u32x4*>(qg + (int64_t)q * p.sq.t + 16 * ks + 8 * g);
      qf[u][ks] = __builtin_bit_cast(vec8<E>, raw);
    }
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (q < Lq) raw = *reinterpret_cast<const u32x4*>(dog + (int64_t)q * p.sdo.t + 16 * ks + 8 * g);
      df[u][ks] = __builtin_bit_cast(vec8<E>, raw);
    }
    lse2[u] = p.lse2[(int64_t)bh * p.Tpad + min(q, p.Tpad - 1)];  // +inf on padding rows
    Dq[u] = q < Lq ? p.D[(int64_t)bh * p.Tpad + q] : 0.f;
  }

  DirectTile<DQ_BN, DQK, BWD_NT / 64> kload;
  DirectTile<DQ_BN, DV, BWD_NT / 64> vload;
  kload.init(skt, w, lane);
  vload.init(svt, w, lane);
  auto load_kv = [&](int key0, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    kload.issue(kg + key0 * skt, skt, Lk - key0, (ATTN_LDS char*)(BUF ? kbuf1 : kbuf0), wu);
    vload.issue(vg + key0 * svt, svt, Lk - key0, (ATTN_LDS char*)(BUF ? vbuf1 : vbuf0), wu);
    if constexpr (KBIAS) {
      if (wu == 0) load_f32x64_lds(p.kbias + (int64_t)bh * p.Tpad + key0, Lk - key0,
                                   (ATTN_LDS float*)(BUF ? kbl1 : kbl0), lane);
    }
  };

  f32x16 dq[QT][NDQ];
#pragma unroll
  for (int u = 0; u < QT; ++u)
#pragma unroll
    for (int t = 0; t < NDQ; ++t) dq[u][t] = zero16();

  // ---- every tile runs as an explicit pipeline (DqPlan).  MASKED: P = 0 on the keys past
  // Lk, past a row's diagonal or under its window (the tiles that carry a mask).  keepr
  // (dropout): keep bits of the rows of query tile u for the tile's 64 keys ----
  using Plan = DqPlan<DQK, DV, QT, KBIAS, DROP>;
  auto tile_pipe = [&](int key0, auto bufc, auto maskc, const u32x2 (&keepr)[QT]) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr bool MASKED = decltype(maskc)::value;
    // key bias of element r of half t: kbv[t][r / 4][r % 4] (score units), read from LDS
    f32x4 kbv[2][4];
    const float* kbl = BUF ? kbl1 : kbl0;
    // dropout: this lane's keep bits of query tile u and half t, shifted by 4 g so that
    // element r sits at bit 8 (r / 4) + r % 4
    uint32_t keepg[QT][2];
#pragma unroll
    for (int u = 0; u < QT; ++u)
#pragma unroll
      for (int t = 0; t < 2; ++t) keepg[u][t] = DROP ? keepr[u][t] >> (4 * g) : 0u;
    // key - query = kq + 32 (t - u) + 8 (r / 4) + r % 4 and Lk - key = lk - 32 t - 8 (r / 4) - r % 4
    // for element r of half t and query tile u
    const int kq = key0 + 4 * g - (qw + lq), lk = Lk - key0 - 4 * g;
    const ATTN_LDS char* kt = (const ATTN_LDS char*)(BUF ? kbuf1 : kbuf0);
    const ATTN_LDS char* vt = (const ATTN_LDS char*)(BUF ? vbuf1 : vbuf0);
    f32x16 s[2][QT], dp[2][QT];
    f32x16 pv[QT];         // P, then dS, of the half being worked on
    // ALiBi: m_h log2(e) (key - query) - LSE log2(e) = abq[u] + ml (32 t + 8 (r / 4) + r % 4)
    // for element r of half t (key key0 + 32 t + 8 (r / 4) + 4 g + r % 4, query qw + 32 u + lq)
    float abq[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u)
      abq[u] = ALIBI ? __builtin_fmaf(ml, (float)(key0 + 4 * g - (qw + 32 * u + lq)), -lse2[u]) : 0.f;
    vec8<E> sb[2][QT][2];
    vec8<E> fr[Plan::RING];
    auto read_at = [&](auto bc) __attribute__((always_inline)) -> vec8<E> {
      constexpr int b = decltype(bc)::value;
      if constexpr (b < Plan::P0)
        return lds_row8<E, DQ_BN>(kt, L, 0, b);
      else if constexpr (b < Plan::S1)
        return lds_row8<E, DQ_BN>(vt, L, 0, b - Plan::P0);
      else if constexpr (b < Plan::P1)
        return lds_row8<E, DQ_BN>(kt, L, 32, b - Plan::S1);
      else if constexpr (b < Plan::Q0)
        return lds_row8<E, DQ_BN>(vt, L, 32, b - Plan::P1);
      else {
        constexpr int t = b < Plan::Q1 ? 0 : 1, jj = b - (t ? Plan::Q1 : Plan::Q0);
        return lds_col8<E, DQ_BN>(kt, L, 32 * t + 16 * (jj % 2), 32 * (jj / 2));
      }
    };
    auto valu_op = [&](auto oc) __attribute__((always_inline)) {
      constexpr int o = decltype(oc)::value, t = Plan::half(o), k = o % (34 * QT);
      if constexpr (Plan::is_p(o)) {
        constexpr int u = k / 16, r = k % 16;
        if constexpr (ALIBI)
          pv[u][r] = exp2_fast(__builtin_fmaf(s[t][u][r], c, __builtin_fmaf(ml, (float)(32 * t + 8 * (r >> 2) + (r & 3)), abq[u])));
        else if constexpr (KBIAS)
          pv[u][r] = exp2_fast(__builtin_fmaf(s[t][u][r], c, __builtin_fmaf(kbv[t][r >> 2][r & 3], c, -lse2[u])));
        else
          pv[u][r] = exp2_fast(__builtin_fmaf(s[t][u][r], c, -lse2[u]));
        if constexpr (MASKED) {
          constexpr int off = 32 * t + 8 * (r >> 2) + (r & 3);
          const int d = kq + off - 32 * u;  // key - query
          pv[u][r] = (off >= lk || (CAUSAL && (d > 0 || (WIN && -d >= W)))) ? 0.f : pv[u][r];
        }
      } else {
        constexpr int kk = k - 16 * QT, u = kk / 18, e = kk % 18;
        if constexpr (e == 8 || e == 17) {
          sb[t][u][e == 8 ? 0 : 1] = pack8<E>(pv[u], e == 8 ? 0 : 1);
        } else {
          constexpr int r = e < 8 ? e : e - 1;
          if constexpr (DROP) {
            // keep bit of element r (bit 8 (r / 4) + r % 4 of this lane's shifted word)
            // spread to all 32 bits, then 1 / (1 - p) or 0 as the multiplier of dP
            constexpr int pos = 8 * (r >> 2) + (r & 3);
            const uint32_t km = (uint32_t)((int32_t)(keepg[u][t] << (31 - pos)) >> 31);
            const float ks = __builtin_bit_cast(float, km & __builtin_bit_cast(uint32_t, p.drop_scale));
            pv[u][r] = pv[u][r] * __builtin_fmaf(dp[t][u][r], ks, -Dq[u]);
          } else {
            pv[u][r] = pv[u][r] * (dp[t][u][r] - Dq[u]);
          }
        }
      }
    };
    static_for<0, Plan::LA>([&](auto bc) __attribute__((always_inline)) { fr[decltype(bc)::value % Plan::RING] = read_at(bc); });
    ATTN_SCHED_FENCE();
    static_for<0, Plan::N>([&](auto bc) __attribute__((always_inline)) {
      constexpr int b = decltype(bc)::value;
      const vec8<E> f = fr[b % Plan::RING];
#pragma unroll
      for (int u = 0; u < QT; ++u) {
        if constexpr (b < Plan::P0)
          s[0][u] = mfma32(f, qf[u][b], b == 0 ? zero16() : s[0][u]);
        else if constexpr (b < Plan::S1)
          dp[0][u] = mfma32(f, df[u][b - Plan::P0], b == Plan::P0 ? zero16() : dp[0][u]);
        else if constexpr (b < Plan::P1)
          s[1][u] = mfma32(f, qf[u][b - Plan::S1], b == Plan::S1 ? zero16() : s[1][u]);
        else if constexpr (b < Plan::Q0)
          dp[1][u] = mfma32(f, df[u][b - Plan::P1], b == Plan::P1 ? zero16() : dp[1][u]);
        else {
          constexpr int t = b < Plan::Q1 ? 0 : 1, jj = b - (t ? Plan::Q1 : Plan::Q0);
          dq[u][jj / 2] = mfma32(f, sb[t][u][jj % 2], dq[u][jj / 2]);
        }
      }
      if constexpr (b + Plan::LA < Plan::N) fr[(b + Plan::LA) % Plan::RING] = read_at(std::integral_constant<int, b + Plan::LA>{});
      if constexpr (KBIAS) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
          if (b == Plan::plan.kb_bundle[t]) {
#pragma unroll
            for (int a = 0; a < 4; ++a) kbv[t][a] = *reinterpret_cast<const f32x4*>(kbl + 32 * t + 8 * a + 4 * g);
          }
      }
      static_for<0, Plan::NOPS>([&](auto oc) __attribute__((always_inline)) {
        if constexpr (Plan::plan.bundle[decltype(oc)::value] == b) valu_op(oc);
      });
      ATTN_SCHED_FENCE();
    });
  };

  // Fixed visiting order: the masked tiles first (those at or above the diagonal or past
  // Lk, then those under the window's lower edge, each descending), then the unmasked
  // ones, descending.  Tiles j >= first_masked hold keys past Lk or past some row's
  // diagonal; tiles j_lo <= j < j_mid hold keys below some row's window.
  const int first_ragged = Lk % DQ_BN != 0 ? Lk / DQ_BN : n_kv;
  const int first_masked = min(min(first_ragged, CAUSAL ? q0 / DQ_BN : n_kv), n_kv);
  const int j_mid = WIN ? max(j_lo, min((max(0, q0 + BM - W) + DQ_BN - 1) / DQ_BN, first_masked)) : j_lo;
  int n_head = n_kv - first_masked;
  int n_msk = n_head + (j_mid - j_lo);
  auto tile_of = [&](int it) {
    if constexpr (BSP) {
      const int u = it + bs_skip;
      return 2 * (bs_idx[u >> 1] & 0xffff) + 1 - (u & 1);
    } else if constexpr (WIN)
      return it < n_head ? n_kv - 1 - it : it < n_msk ? j_mid - 1 - (it - n_head) : first_masked - 1 - (it - n_msk);
    else
      return n_kv - 1 - it;
  };
  if constexpr (BSP) {  // the masked tiles are the highest ones, so they lead the list
    n_head = 0;
    while (n_head < n_tiles && tile_of(n_head) >= first_masked) ++n_head;
    n_msk = n_head;
  }
  load_kv(tile_of(0) * DQ_BN, std::integral_constant<int, 0>{});
  auto step = [&](int it, auto bufc, auto maskc) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;
    const int j = tile_of(it);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // dropout keep bits of this lane's rows for keys 64 j .. 64 j + 63, read before the next
    // tile's loads
    u32x2 keepr[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      keepr[u] = u32x2{0u, 0u};
      if constexpr (DROP)
        keepr[u] = *reinterpret_cast<const u32x2*>(  // rows past the mask's are padding (P = 0)
            p.drop_rows + ((int64_t)bh * p.drop_tp + min(qw + 32 * u + lq, p.drop_tp - 1)) * p.drop_ld + j * (DQ_BN / 8));
    }
    if (it + 1 < n_tiles) load_kv(tile_of(it + 1) * DQ_BN, std::integral_constant<int, 1 - BUF>{});
    const int key0 = j * DQ_BN;
    if (BSP && ((bs_idx[(it + bs_skip) >> 1] >> bs_row) & 1) == 0) return;  // no live block for these rows
    if constexpr (decltype(maskc)::value) {
      if (CAUSAL && key0 > qw + 32 * QT - 1) return;  // tile wholly above this wavefront's rows
      if (WIN && key0 + DQ_BN <= qw - W + 1) return;  // tile wholly below its rows' windows
      const bool need = (CAUSAL && (key0 + DQ_BN - 1 > qw || (WIN && key0 < qw + 32 * QT - W))) || key0 + DQ_BN > Lk;
      if (need)
        tile_pipe(key0, bufc, std::true_type{}, keepr);
      else
        tile_pipe(key0, bufc, std::false_type{}, keepr);
    } else {
      tile_pipe(key0, bufc, std::false_type{}, keepr);
    }
  };
  // The first tiles (the workgroup's diagonal ones under the causal mask, or the ragged
  // last key block) may carry a mask for some wavefront; they run as the pipeline's
  // masked form, the rest as its unmasked form.
  constexpr auto B0 = std::integral_constant<int, 0>{};
  constexpr auto B1 = std::integral_constant<int, 1>{};
  int it = 0;
  for (; it < n_msk; ++it) {
    if (it & 1)
      step(it, B1, std::true_type{});
    else
      step(it, B0, std::true_type{});
  }
  if ((it & 1) && it < n_tiles) step(it++, B1, std::false_type{});
  for (; it + 1 < n_tiles; it += 2) {
    step(it, B0, std::false_type{});
    step(it + 1, B1, std::false_type{});
  }
  if (it < n_tiles) step(it, B0, std::false_type{});

#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int q = qw + 32 * u + lq;
    if (q < T) {
      E* row = dqg + (int64_t)q * p.sdq.t;
#pragma unroll
      for (int t = 0; t < NDQ; ++t)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          vec4<E> v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (E)(dq[u][t][4 * a + e] * p.scale);
          *reinterpret_cast<vec4<E>*>(row + 32 * t + 8 * a + 4 * g) = v;
        }
    }
  }
}

template <class E, int DQK, int DV, bool CAUSAL, bool WIN, bool ALIBI, bool BSP = false, bool KBIAS = false,
          bool DROP = false>
__global__ __launch_bounds__(BWD_NT) __attribute__((amdgpu_waves_per_eu(DqShape<DQK>::WAVES_PER_EU,
                                                                         DqShape<DQK>::WAVES_PER_EU)))
void bwd_dq_kernel(BwdParams p) {
  bwd_dq_body<E, DQK, DV, CAUSAL, WIN, ALIBI, BSP, KBIAS, DROP>(p, (int)blockIdx.x);
}

// ---------------------------------------------------------------------------------
// finalize: dQ = scale * accumulator -> bf16
// ---------------------------------------------------------------------------------
template <class E, int DQK>
__global__ __launch_bounds__(256) void bwd_finalize_kernel(BwdParams p) {
  constexpr int G = DQK / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / G;
  const int c = (int)(gid % G);
  if (row >= (int64_t)p.B * p.NH * p.Tpad) return;
  const int t = (int)(row % p.Tpad);
  if (t >= p.T) return;
  const int bh = (int)(row / p.Tpad);
  const int b = bh / p.NH, h = bh % p.NH;
  const float* src = p.dq_acc + row * DQK + 8 * c;
  const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
  const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
  vec8<E> v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = (E)(x0[e] * p.scale);
    v[4 + e] = (E)(x1[e] * p.scale);
  }
  E* dst = (E*)p.dq + b * p.sdq.b + h * p.sdq.h + (int64_t)t * p.sdq.t + 8 * c;
  *reinterpret_cast<u32x4*>(dst) = __builtin_bit_cast(u32x4, v);
}

// ---------------------------------------------------------------------------------
// per-configuration launchers (each instantiated by one compilation of attn_bwd_inst.hip)
// ---------------------------------------------------------------------------------
// MASK: 0 none, 1 causal, 2 causal with a sliding window of p.win keys, 3 causal with the
// ALiBi bias, 4 block-sparse map, 5 block-sparse map and causal, 6 key bias, 7 key bias
// and causal.
// MASK 4: block-sparse map; 5: block-sparse map and the causal mask; 6: key bias;
// 7: key bias and the causal mask; 8: dropout; 9: dropout and the causal mask.
template <int MASK>
struct MaskMode {
  static constexpr bool CAUSAL = MASK == 1 || MASK == 2 || MASK == 3 || MASK == 5 || MASK == 7 || MASK == 9;
  static constexpr bool WIN = MASK == 2, ALIBI = MASK == 3, BSP = MASK == 4 || MASK == 5;
  static constexpr bool KBIAS = MASK == 6 || MASK == 7, DROP = MASK == 8 || MASK == 9;
};

template <class E, int DQK, int DV, int MASK>
hipError_t bwd_main_t(const BwdParams& p, bool deterministic, hipStream_t s) {
  using M = MaskMode<MASK>;
  const int nkb = (p.T + BWD_BN - 1) / BWD_BN;
  const dim3 grid_kv(nkb * p.B * p.NH);
  if (deterministic)
    hipLaunchKernelGGL((bwd_kv_kernel<E, DQK, DV, M::CAUSAL, M::WIN, M::ALIBI, false, M::BSP, M::KBIAS, M::DROP>), grid_kv,
                       dim3(BWD_NT), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_kv_kernel<E, DQK, DV, M::CAUSAL, M::WIN, M::ALIBI, true, M::BSP, M::KBIAS, M::DROP>), grid_kv,
                       dim3(BWD_NT), 0, s, p);
  return hipGetLastError();
}

template <class E, int DQK, int DV, int MASK>
hipError_t bwd_dq_t(const BwdParams& p, hipStream_t s) {
  using M = MaskMode<MASK>;
  const int nqb = (p.T + DqShape<DQK>::BM - 1) / DqShape<DQK>::BM;
  hipLaunchKernelGGL((bwd_dq_kernel<E, DQK, DV, M::CAUSAL, M::WIN, M::ALIBI, M::BSP, M::KBIAS, M::DROP>),
                     dim3(nqb * p.B * p.NH), dim3(BWD_NT), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// d = 64, deterministic mode: the key/value and dQ work items in one launch
// ---------------------------------------------------------------------------------
// The two kernels read only the inputs and the preprocess output, so their work items
// may run side by side.  At short sequences neither grid fills the GPU by itself (384 +
// 384 workgroups at the GPT-2 shape against 512 resident slots) and each launch ends in a
// tail; one launch lets the dQ items fill the slots the key/value items leave.  The first
// nkv workgroups run the key/value items and the rest the dQ items, each set in its own
// longest-first order (padded batches: the planner's work lists); nkv is a multiple of 8,
// so both orders keep their XCD grouping.
// At d = 64 both bodies run at two wavefronts per SIMD, and their LDS tiles together
// still fit two workgroups per CU.
template <class E, bool CAUSAL>
__global__ __launch_bounds__(BWD_NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_kvdq64_kernel(BwdParams p,
                                                                                                        int nkv) {
  if ((int)blockIdx.x < nkv)
    bwd_kv_body<E, 64, 64, CAUSAL, false, false, false>(p, (int)blockIdx.x);
  else
    bwd_dq_body<E, 64, 64, CAUSAL, false, false>(p, (int)blockIdx.x - nkv);
}

// Workgroups of the key/value and dQ launches at d = 64; the merged launch needs nkv % 8 == 0.
inline int kvdq64_nkv(const BwdParams& p) { return (p.T + BWD_BN - 1) / BWD_BN * p.B * p.NH; }
inline int kvdq64_ndq(const BwdParams& p) { return (p.T + DqShape<64>::BM - 1) / DqShape<64>::BM * p.B * p.NH; }

template <class E, int MASK>
hipError_t bwd_kvdq64_t(const BwdParams& p, hipStream_t s) {
  static_assert(MASK == 0 || MASK == 1, "the merged launch serves the plain and causal masks only");
  const int nkv = kvdq64_nkv(p);
  hipLaunchKernelGGL((bwd_kvdq64_kernel<E, MASK == 1>), dim3(nkv + kvdq64_ndq(p)), dim3(BWD_NT), 0, s, p, nkv);
  return hipGetLastError();
}

#define ATTN_BWD_CONFIGS(X)                                                                        \
  X(64, 64, 0) X(64, 64, 1) X(64, 64, 2) X(64, 64, 3) X(128, 128, 0) X(128, 128, 1) X(128, 128, 2) \
  X(128, 128, 3) X(192, 128, 0) X(192, 128, 1) X(192, 128, 2) X(192, 128, 3)
#define ATTN_EXTERN_BWD_E(E, DQK, DV, MASK)                                                       \
  extern template hipError_t bwd_main_t<E, DQK, DV, MASK>(const BwdParams&, bool, hipStream_t); \
  extern template hipError_t bwd_dq_t<E, DQK, DV, MASK>(const BwdParams&, hipStream_t);
#define ATTN_EXTERN_BWD(DQK, DV, MASK) ATTN_EXTERN_BWD_E(bf16, DQK, DV, MASK) ATTN_EXTERN_BWD_E(f16, DQK, DV, MASK)
ATTN_BWD_CONFIGS(ATTN_EXTERN_BWD)
// block-sparse maps, the key bias and dropout: bf16 only
#define ATTN_BWD_BSP_CONFIGS(X)                                                                       \
  X(64, 64, 4) X(64, 64, 5) X(128, 128, 4) X(128, 128, 5) X(192, 128, 4) X(192, 128, 5) X(64, 64, 6) \
  X(64, 64, 7) X(128, 128, 6) X(128, 128, 7) X(192, 128, 6) X(192, 128, 7) X(64, 64, 8) X(64, 64, 9) X(128, 128, 8) \
  X(128, 128, 9) X(192, 128, 8) X(192, 128, 9)
#define ATTN_EXTERN_BWD_BF16(DQK, DV, MASK) ATTN_EXTERN_BWD_E(bf16, DQK, DV, MASK)
ATTN_BWD_BSP_CONFIGS(ATTN_EXTERN_BWD_BF16)
extern template hipError_t bwd_kvdq64_t<bf16, 0>(const BwdParams&, hipStream_t);
extern template hipError_t bwd_kvdq64_t<bf16, 1>(const BwdParams&, hipStream_t);
extern template hipError_t bwd_kvdq64_t<f16, 0>(const BwdParams&, hipStream_t);
extern template hipError_t bwd_kvdq64_t<f16, 1>(const BwdParams&, hipStream_t);

}  // namespace attn53
