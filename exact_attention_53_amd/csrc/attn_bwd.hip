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
//                      P_ij dP_ij = P_ij sum_k dO_ik V_jk over j gives sum_k dO_ik O_ik);
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
#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn53 {

constexpr int BWD_BN = 128;  // keys per workgroup (32 per wavefront)
constexpr int BWD_BM = 64;   // queries per step
constexpr int BWD_NT = 256;
constexpr int DQ_BM = 128;   // deterministic dQ kernel: queries per workgroup
constexpr int DQ_BN = 64;    //                           keys per step

// ---------------------------------------------------------------------------------
// preprocess: D = rowsum(dO * O); optional clear of the dQ accumulator
// ---------------------------------------------------------------------------------
template <int DV>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int d_qk, int zero_acc) {
  constexpr int G = DV / 8;  // lanes per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / G;  // over B * NH * Tpad
  const int c = (int)(gid % G);
  const int64_t nrows = (int64_t)p.B * p.NH * p.Tpad;
  float sum = 0.f;
  if (row < nrows) {
    const int t = (int)(row % p.Tpad);
    const int bh = (int)(row / p.Tpad);
    const int b = bh / p.NH, h = bh % p.NH;
    if (t < p.T) {
      const bf16* orow = (const bf16*)p.o + b * p.so.b + h * p.so.h + (int64_t)t * p.so.t;
      const bf16* drow = (const bf16*)p.dO + b * p.sdo.b + h * p.sdo.h + (int64_t)t * p.sdo.t;
      const bf16x8 ov = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(orow + 8 * c));
      const bf16x8 dv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(drow + 8 * c));
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += (float)ov[e] * (float)dv[e];
    }
    if (zero_acc) {
      float* acc = p.dq_acc + row * d_qk;
      for (int x = 4 * c; x < d_qk; x += 4 * G) *reinterpret_cast<f32x4*>(acc + x) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, G);
  if (row < nrows && c == 0) p.D[row] = sum;
}

// ---------------------------------------------------------------------------------
// main backward: key/value-stationary
// ---------------------------------------------------------------------------------
template <int DQK, int DV, bool CAUSAL, bool ATOMIC_DQ>
__global__ __launch_bounds__(BWD_NT) void bwd_kv_kernel(BwdParams p) {
  constexpr int KSQ = DQK / 16, KSV = DV / 16;
  constexpr int NDK = DQK / 32, NDV = DV / 32;
  constexpr int NDQ = DQK / 32 / 2;                     // dQ tiles per wavefront
  constexpr int QT_BYTES = BWD_BM * DQK * 2;            // Q tile
  constexpr int OT_BYTES = BWD_BM * DV * 2;             // dO tile
  constexpr int KD_BYTES = ATOMIC_DQ ? BWD_BN * DQK * 2 : 0;   // K block for dQ = dS K
  constexpr int ST_BYTES = ATOMIC_DQ ? BWD_BN * BWD_BM * 2 : 0;  // dS^T tile
  constexpr int OFF_Q = 0;
  constexpr int OFF_O = OFF_Q + 2 * QT_BYTES;
  constexpr int OFF_K = OFF_O + 2 * OT_BYTES;
  constexpr int OFF_S = OFF_K + KD_BYTES;
  constexpr int OFF_L = OFF_S + ST_BYTES;                // lse*log2e and D, 2 buffers
  constexpr int LDS_BYTES = OFF_L + 2 * 2 * BWD_BM * 4;
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  ATTN_LDS char* lds = (ATTN_LDS char*)smem;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, lq = lane & 31;
  const int T = p.T;
  const int nkb = (T + BWD_BN - 1) / BWD_BN;
  const int nqb = (T + BWD_BM - 1) / BWD_BM;
  const Item item = schedule(blockIdx.x, p.B * p.NH);
  const int kb = item.rank;  // causal: block 0 has the most query blocks -> first
  const int b = item.bh / p.NH, h = item.bh % p.NH;

  const bf16* qg = (const bf16*)p.q + b * p.sq.b + h * p.sq.h;
  const bf16* kg = (const bf16*)p.k + b * p.sk.b + h * p.sk.h;
  const bf16* vg = (const bf16*)p.v + b * p.sv.b + h * p.sv.h;
  const bf16* dog = (const bf16*)p.dO + b * p.sdo.b + h * p.sdo.h;
  const float* lseg = p.lse + (int64_t)item.bh * T;
  const float* Dg = p.D + (int64_t)item.bh * p.Tpad;
  float* dqacc = p.dq_acc + (int64_t)item.bh * p.Tpad * DQK;
  (void)nkb;

  const int key0 = kb * BWD_BN;
  const int kw = 32 * w;
  const int my_key = key0 + kw + lq;

  // K and V rows of this wavefront as B-operand fragments of S = Q K^T and dP = dO V^T.
  bf16x8 kf[KSQ], vf[KSV];
#pragma unroll
  for (int ks = 0; ks < KSQ; ++ks) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (my_key < T) raw = *reinterpret_cast<const u32x4*>(kg + (int64_t)my_key * p.sk.t + 16 * ks + 8 * g);
    kf[ks] = __builtin_bit_cast(bf16x8, raw);
  }
#pragma unroll
  for (int ks = 0; ks < KSV; ++ks) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (my_key < T) raw = *reinterpret_cast<const u32x4*>(vg + (int64_t)my_key * p.sv.t + 16 * ks + 8 * g);
    vf[ks] = __builtin_bit_cast(bf16x8, raw);
  }

  const int i0 = CAUSAL ? key0 / BWD_BM : 0;
  const int n_q = nqb - i0;

  TileStage<BWD_BM, DQK, BWD_NT> qst;
  TileStage<BWD_BM, DV, BWD_NT> ost;
  float lsev = 0.f, dval = 0.f;  // threads 0..63: LSE*log2e, threads 64..127: D
  auto load_rows = [&](int qb) {
    qst.load(qg, p.sq.t, qb * BWD_BM, T, tid);
    ost.load(dog, p.sdo.t, qb * BWD_BM, T, tid);
    const int r = qb * BWD_BM + (tid & 63);
    if (tid < 64) lsev = r < T ? lseg[r] * kLog2e : INFINITY;  // rows >= T: P = 0
    else if (tid < 128) dval = r < T ? Dg[r] : 0.f;
  };
  auto store_rows = [&](int buf) {
    qst.store(lds + OFF_Q + buf * QT_BYTES, tid);
    ost.store(lds + OFF_O + buf * OT_BYTES, tid);
    float* lb = (float*)(smem + OFF_L + buf * 2 * BWD_BM * 4);
    if (tid < 64) lb[tid] = lsev;
    else if (tid < 128) lb[BWD_BM + tid - 64] = dval;
  };

  if (ATOMIC_DQ) {
    TileStage<BWD_BN, DQK, BWD_NT> kst;
    kst.load(kg, p.sk.t, key0, T, tid);
    kst.store(lds + OFF_K, tid);
  }
  load_rows(i0);
  store_rows(0);
  __syncthreads();

  f32x16 dk[NDK], dv[NDV];
#pragma unroll
  for (int t = 0; t < NDK; ++t) dk[t] = zero16();
#pragma unroll
  for (int t = 0; t < NDV; ++t) dv[t] = zero16();

  for (int it = 0; it < n_q; ++it) {
    const int qb = i0 + it;
    const int buf = it & 1;
    const bool more = it + 1 < n_q;
    if (more) load_rows(qb + 1);
    const int q0 = qb * BWD_BM;
    const ATTN_LDS char* qt = lds + OFF_Q + buf * QT_BYTES;
    const ATTN_LDS char* ot = lds + OFF_O + buf * OT_BYTES;
    const float* lb = (const float*)(smem + OFF_L + buf * 2 * BWD_BM * 4);

    // S = Q K^T and dP = dO V^T for 64 queries x this wavefront's 32 keys
    f32x16 s[2], dp[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = zero16();
      dp[t] = zero16();
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks) s[t] = mfma32(lds_row8<BWD_BM>(qt, 32 * t + lq, 16 * ks + 8 * g), kf[ks], s[t]);
#pragma unroll
      for (int ks = 0; ks < KSV; ++ks) dp[t] = mfma32(lds_row8<BWD_BM>(ot, 32 * t + lq, 16 * ks + 8 * g), vf[ks], dp[t]);
    }
    // P = 2^(S scale log2e - LSE log2e), dS = P (dP - D); element r of tile t is
    // query q0 + 32 t + 8 (r / 4) + 4 g + r % 4, key my_key.
    const bool need_mask = (CAUSAL && key0 + BWD_BN - 1 > q0) || (key0 + BWD_BN > T) || (q0 + BWD_BM > T);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int qi = 32 * t + 8 * a + 4 * g;
        const f32x4 L = *reinterpret_cast<const f32x4*>(lb + qi);
        const f32x4 Dd = *reinterpret_cast<const f32x4*>(lb + BWD_BM + qi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * a + e;
          float pv = exp2_fast(s[t][r] * p.scale_log2 - L[e]);
          if (need_mask) {
            const int q = q0 + qi + e;
            if (my_key >= T || q >= T || (CAUSAL && my_key > q)) pv = 0.f;
          }
          s[t][r] = pv;
          dp[t][r] = pv * (dp[t][r] - Dd[e]);
        }
      }
    const bf16x8 pb[4] = {pack8(s[0], 0), pack8(s[0], 1), pack8(s[1], 0), pack8(s[1], 1)};
    const bf16x8 sb[4] = {pack8(dp[0], 0), pack8(dp[0], 1), pack8(dp[1], 0), pack8(dp[1], 1)};
    // dV += P^T dO,  dK += dS^T Q   (contraction over the 64 queries)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int t = 0; t < NDV; ++t) dv[t] = mfma32(pb[m], lds_col8<BWD_BM>(ot, 16 * m, 32 * t, lane), dv[t]);
#pragma unroll
      for (int t = 0; t < NDK; ++t) dk[t] = mfma32(sb[m], lds_col8<BWD_BM>(qt, 16 * m, 32 * t, lane), dk[t]);
    }
    if constexpr (ATOMIC_DQ) {
      // dS^T tile in LDS: row = key (128), column = query (64)
      ATTN_LDS char* st = lds + OFF_S;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (bf16)dp[t][4 * a + e];
          *reinterpret_cast<ATTN_LDS bf16x4*>(st + tile_off<BWD_BN>(kw + lq, 32 * t + 8 * a + 4 * g)) = v;
        }
      __syncthreads();
      // partial dQ (64 x DQK) = dS K over this block's 128 keys; wavefront w owns query
      // tile w % 2 and d tiles (w / 2) * NDQ .. +NDQ-1
      const int tq = w & 1;
      f32x16 dq[NDQ];
#pragma unroll
      for (int n = 0; n < NDQ; ++n) dq[n] = zero16();
      const ATTN_LDS char* kd = lds + OFF_K;
#pragma unroll
      for (int m = 0; m < BWD_BN / 16; ++m) {
        const bf16x8 a = lds_col8<BWD_BN>(st, 16 * m, 32 * tq, lane);
#pragma unroll
        for (int n = 0; n < NDQ; ++n)
          dq[n] = mfma32(a, lds_col8<BWD_BN>(kd, 16 * m, 32 * ((w >> 1) * NDQ + n), lane), dq[n]);
      }
#pragma unroll
      for (int n = 0; n < NDQ; ++n) {
        const int d = 32 * ((w >> 1) * NDQ + n) + lq;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + 32 * tq + 8 * (r >> 2) + 4 * g + (r & 3);  // < Tpad
          unsafeAtomicAdd(dqacc + (int64_t)q * DQK + d, dq[n][r]);
        }
      }
    }
    if (more) store_rows(buf ^ 1);
    __syncthreads();
  }

  // dK = scale dS^T Q, dV; element r of tile t: key key0 + kw + 8 (r / 4) + 4 g + r % 4,
  // column 32 t + lq.
  bf16* dkg = (bf16*)p.dk + b * p.sdk.b + h * p.sdk.h;
  bf16* dvg = (bf16*)p.dv + b * p.sdv.b + h * p.sdv.h;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = key0 + kw + 8 * (r >> 2) + 4 * g + (r & 3);
    if (key < T) {
#pragma unroll
      for (int t = 0; t < NDK; ++t) dkg[(int64_t)key * p.sdk.t + 32 * t + lq] = (bf16)(dk[t][r] * p.scale);
#pragma unroll
      for (int t = 0; t < NDV; ++t) dvg[(int64_t)key * p.sdv.t + 32 * t + lq] = (bf16)dv[t][r];
    }
  }
}

// ---------------------------------------------------------------------------------
// deterministic dQ: query-stationary, fixed key-block order
// ---------------------------------------------------------------------------------
template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__(BWD_NT) void bwd_dq_kernel(BwdParams p) {
  constexpr int KSQ = DQK / 16, KSV = DV / 16, NDQ = DQK / 32;
  constexpr int KT_BYTES = DQ_BN * DQK * 2;
  constexpr int VT_BYTES = DQ_BN * DV * 2;
  __shared__ __attribute__((aligned(16))) char smem[2 * (KT_BYTES + VT_BYTES)];
  ATTN_LDS char* lds = (ATTN_LDS char*)smem;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, lq = lane & 31;
  const int T = p.T;
  const int nqb = (T + DQ_BM - 1) / DQ_BM;
  const Item item = schedule(blockIdx.x, p.B * p.NH);
  const int qb = CAUSAL ? nqb - 1 - item.rank : item.rank;
  const int b = item.bh / p.NH, h = item.bh % p.NH;

  const bf16* qg = (const bf16*)p.q + b * p.sq.b + h * p.sq.h;
  const bf16* kg = (const bf16*)p.k + b * p.sk.b + h * p.sk.h;
  const bf16* vg = (const bf16*)p.v + b * p.sv.b + h * p.sv.h;
  const bf16* dog = (const bf16*)p.dO + b * p.sdo.b + h * p.sdo.h;
  bf16* dqg = (bf16*)p.dq + b * p.sdq.b + h * p.sdq.h;

  const int q0 = qb * DQ_BM, qw = q0 + 32 * w, my_q = qw + lq;

  // Q and dO rows as B operands of S^T = K Q^T and dP^T = V dO^T
  bf16x8 qf[KSQ], df[KSV];
#pragma unroll
  for (int ks = 0; ks < KSQ; ++ks) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (my_q < T) raw = *reinterpret_cast<const u32x4*>(qg + (int64_t)my_q * p.sq.t + 16 * ks + 8 * g);
    qf[ks] = __builtin_bit_cast(bf16x8, raw);
  }
#pragma unroll
  for (int ks = 0; ks < KSV; ++ks) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (my_q < T) raw = *reinterpret_cast<const u32x4*>(dog + (int64_t)my_q * p.sdo.t + 16 * ks + 8 * g);
    df[ks] = __builtin_bit_cast(bf16x8, raw);
  }
  const float lse2 = my_q < T ? p.lse[(int64_t)item.bh * T + my_q] * kLog2e : INFINITY;
  const float Dq = my_q < T ? p.D[(int64_t)item.bh * p.Tpad + my_q] : 0.f;

  const int kv_end = CAUSAL ? min(T, q0 + DQ_BM) : T;
  const int n_kv = (kv_end + DQ_BN - 1) / DQ_BN;

  TileStage<DQ_BN, DQK, BWD_NT> kst;
  TileStage<DQ_BN, DV, BWD_NT> vst;
  kst.load(kg, p.sk.t, (n_kv - 1) * DQ_BN, T, tid);
  vst.load(vg, p.sv.t, (n_kv - 1) * DQ_BN, T, tid);
  kst.store(lds, tid);
  vst.store(lds + 2 * KT_BYTES, tid);
  __syncthreads();

  f32x16 dq[NDQ];
#pragma unroll
  for (int t = 0; t < NDQ; ++t) dq[t] = zero16();

  for (int it = 0; it < n_kv; ++it) {
    const int j = n_kv - 1 - it;  // fixed order: descending key block
    const int buf = it & 1;
    const bool more = it + 1 < n_kv;
    if (more) {
      kst.load(kg, p.sk.t, (j - 1) * DQ_BN, T, tid);
      vst.load(vg, p.sv.t, (j - 1) * DQ_BN, T, tid);
    }
    const int key0 = j * DQ_BN;
    const bool active = !CAUSAL || key0 <= qw + 31;
    if (active) {
      const ATTN_LDS char* kt = lds + buf * KT_BYTES;
      const ATTN_LDS char* vt = lds + 2 * KT_BYTES + buf * VT_BYTES;
      f32x16 s[2], dp[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s[t] = zero16();
        dp[t] = zero16();
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks) s[t] = mfma32(lds_row8<DQ_BN>(kt, 32 * t + lq, 16 * ks + 8 * g), qf[ks], s[t]);
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) dp[t] = mfma32(lds_row8<DQ_BN>(vt, 32 * t + lq, 16 * ks + 8 * g), df[ks], dp[t]);
      }
      const bool need_mask = (CAUSAL && key0 + DQ_BN - 1 > qw) || (key0 + DQ_BN > T);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = exp2_fast(s[t][r] * p.scale_log2 - lse2);
          if (need_mask) {
            const int key = key0 + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= T || (CAUSAL && key > my_q)) pv = 0.f;
          }
          dp[t][r] = pv * (dp[t][r] - Dq);
        }
      const bf16x8 sb[4] = {pack8(dp[0], 0), pack8(dp[0], 1), pack8(dp[1], 0), pack8(dp[1], 1)};
      // dQ^T += K^T dS^T
#pragma unroll
      for (int t = 0; t < NDQ; ++t)
#pragma unroll
        for (int m = 0; m < 4; ++m) dq[t] = mfma32(lds_col8<DQ_BN>(kt, 16 * m, 32 * t, lane), sb[m], dq[t]);
    }
    if (more) {
      kst.store(lds + (buf ^ 1) * KT_BYTES, tid);
      vst.store(lds + 2 * KT_BYTES + (buf ^ 1) * VT_BYTES, tid);
    }
    __syncthreads();
  }

  if (my_q < T) {
    bf16* row = dqg + (int64_t)my_q * p.sdq.t;
#pragma unroll
    for (int t = 0; t < NDQ; ++t)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(dq[t][4 * a + e] * p.scale);
        *reinterpret_cast<bf16x4*>(row + 32 * t + 8 * a + 4 * g) = v;
      }
  }
}

// ---------------------------------------------------------------------------------
// finalize: dQ = scale * accumulator -> bf16
// ---------------------------------------------------------------------------------
template <int DQK>
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
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = (bf16)(x0[e] * p.scale);
    v[4 + e] = (bf16)(x1[e] * p.scale);
  }
  bf16* dst = (bf16*)p.dq + b * p.sdq.b + h * p.sdq.h + (int64_t)t * p.sdq.t + 8 * c;
  *reinterpret_cast<u32x4*>(dst) = __builtin_bit_cast(u32x4, v);
}

// ---------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------
static inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

hipError_t launch_bwd_preprocess(const BwdParams& p, int d_qk, int d_v, bool zero_acc, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.NH * p.Tpad;
  if (d_v == 64)
    hipLaunchKernelGGL((bwd_pre_kernel<64>), dim3(blocks_for(rows * 8)), dim3(256), 0, s, p, d_qk, (int)zero_acc);
  else if (d_v == 128)
    hipLaunchKernelGGL((bwd_pre_kernel<128>), dim3(blocks_for(rows * 16)), dim3(256), 0, s, p, d_qk, (int)zero_acc);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int DQK, int DV, bool CAUSAL>
static hipError_t bwd_main_t(const BwdParams& p, bool deterministic, hipStream_t s) {
  const int nkb = (p.T + BWD_BN - 1) / BWD_BN;
  const dim3 grid_kv(nkb * p.B * p.NH);
  if (deterministic) {
    hipLaunchKernelGGL((bwd_kv_kernel<DQK, DV, CAUSAL, false>), grid_kv, dim3(BWD_NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nqb = (p.T + DQ_BM - 1) / DQ_BM;
    hipLaunchKernelGGL((bwd_dq_kernel<DQK, DV, CAUSAL>), dim3(nqb * p.B * p.NH), dim3(BWD_NT), 0, s, p);
  } else {
    hipLaunchKernelGGL((bwd_kv_kernel<DQK, DV, CAUSAL, true>), grid_kv, dim3(BWD_NT), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_main(const BwdParams& p, int d_qk, int d_v, bool causal, bool deterministic, hipStream_t s) {
  if (d_qk == 64 && d_v == 64)
    return causal ? bwd_main_t<64, 64, true>(p, deterministic, s) : bwd_main_t<64, 64, false>(p, deterministic, s);
  if (d_qk == 128 && d_v == 128)
    return causal ? bwd_main_t<128, 128, true>(p, deterministic, s) : bwd_main_t<128, 128, false>(p, deterministic, s);
  if (d_qk == 192 && d_v == 128)
    return causal ? bwd_main_t<192, 128, true>(p, deterministic, s) : bwd_main_t<192, 128, false>(p, deterministic, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_finalize(const BwdParams& p, int d_qk, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.NH * p.Tpad;
  if (d_qk == 64)
    hipLaunchKernelGGL((bwd_finalize_kernel<64>), dim3(blocks_for(rows * 8)), dim3(256), 0, s, p);
  else if (d_qk == 128)
    hipLaunchKernelGGL((bwd_finalize_kernel<128>), dim3(blocks_for(rows * 16)), dim3(256), 0, s, p);
  else if (d_qk == 192)
    hipLaunchKernelGGL((bwd_finalize_kernel<192>), dim3(blocks_for(rows * 24)), dim3(256), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace attn53
