// Exact attention backward for gfx950: launchers of the preprocess and finalize
// kernels and dispatch of the per-configuration key/value and dQ launchers.  The
// kernels themselves are in attn_bwd_kernels.hpp.
#include <type_traits>

#include "attn_bwd_kernels.hpp"

namespace attn53 {

// ---------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------
static inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

template <class E>
static hipError_t pre_t(const BwdParams& p, int d_qk, int d_v, bool zero_acc, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.NH * p.Tpad;
  // a workgroup covers NP * 256 / G rows, G = d_v / 8 lanes per row; four rows per lane
  // group where that still leaves at least 2048 workgroups (8 per CU)
  const int64_t lanes = rows * (d_v / 8);
  const bool wide = blocks_for(lanes / 4) >= 2048;
  if (d_v == 64 && wide)
    hipLaunchKernelGGL((bwd_pre_kernel<E, 64, 4>), dim3(blocks_for(lanes / 4)), dim3(256), 0, s, p, d_qk, (int)zero_acc);
  else if (d_v == 64)
    hipLaunchKernelGGL((bwd_pre_kernel<E, 64, 1>), dim3(blocks_for(lanes)), dim3(256), 0, s, p, d_qk, (int)zero_acc);
  else if (d_v == 128 && wide)
    hipLaunchKernelGGL((bwd_pre_kernel<E, 128, 4>), dim3(blocks_for(lanes / 4)), dim3(256), 0, s, p, d_qk, (int)zero_acc);
  else if (d_v == 128)
    hipLaunchKernelGGL((bwd_pre_kernel<E, 128, 1>), dim3(blocks_for(lanes)), dim3(256), 0, s, p, d_qk, (int)zero_acc);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_preprocess(const BwdParams& p, ElemType et, int d_qk, int d_v, bool zero_acc, hipStream_t s) {
  return et == ELEM_F16 ? pre_t<f16>(p, d_qk, d_v, zero_acc, s) : pre_t<bf16>(p, d_qk, d_v, zero_acc, s);
}

// mask mode of the launchers: 0 none, 1 causal, 2 causal with a sliding window, 3 causal
// with the ALiBi bias, 4 block-sparse map, 5 block-sparse map and causal, 6 key bias,
// 7 key bias and causal, 8 dropout, 9 dropout and causal
static inline int mask_mode(const BwdParams& p, bool causal) {
  if (p.bsp) return causal ? 5 : 4;
  if (p.kbias != nullptr) return causal ? 7 : 6;
  if (p.drop_rows != nullptr) return causal ? 9 : 8;
  return !causal ? 0 : p.win < kNoWindow ? 2 : p.alibi ? 3 : 1;
}

template <class E, int DQK, int DV>
static hipError_t main_m(const BwdParams& p, bool causal, bool det, hipStream_t s) {
  switch (mask_mode(p, causal)) {
    case 0: return bwd_main_t<E, DQK, DV, 0>(p, det, s);
    case 1: return bwd_main_t<E, DQK, DV, 1>(p, det, s);
    case 2: return bwd_main_t<E, DQK, DV, 2>(p, det, s);
    case 3: return bwd_main_t<E, DQK, DV, 3>(p, det, s);
    default:
      if constexpr (std::is_same<E, bf16>::value) {  // block-sparse maps and the key bias: bf16 only
        switch (mask_mode(p, causal)) {
          case 4: return bwd_main_t<E, DQK, DV, 4>(p, det, s);
          case 5: return bwd_main_t<E, DQK, DV, 5>(p, det, s);
          case 6: return bwd_main_t<E, DQK, DV, 6>(p, det, s);
          case 7: return bwd_main_t<E, DQK, DV, 7>(p, det, s);
          case 8: return bwd_main_t<E, DQK, DV, 8>(p, det, s);
          default: return bwd_main_t<E, DQK, DV, 9>(p, det, s);
        }
      } else {
        return hipErrorInvalidValue;
      }
  }
}

template <class E>
static hipError_t main_t(const BwdParams& p, int d_qk, int d_v, bool causal, bool det, hipStream_t s) {
  if (d_qk == 64 && d_v == 64) return main_m<E, 64, 64>(p, causal, det, s);
  if (d_qk == 128 && d_v == 128) return main_m<E, 128, 128>(p, causal, det, s);
  if (d_qk == 192 && d_v == 128) return main_m<E, 192, 128>(p, causal, det, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_main(const BwdParams& p, ElemType et, int d_qk, int d_v, bool causal, bool deterministic,
                           hipStream_t s) {
  return et == ELEM_F16 ? main_t<f16>(p, d_qk, d_v, causal, deterministic, s)
                        : main_t<bf16>(p, d_qk, d_v, causal, deterministic, s);
}

template <class E, int DQK, int DV>
static hipError_t dq_m(const BwdParams& p, bool causal, hipStream_t s) {
  switch (mask_mode(p, causal)) {
    case 0: return bwd_dq_t<E, DQK, DV, 0>(p, s);
    case 1: return bwd_dq_t<E, DQK, DV, 1>(p, s);
    case 2: return bwd_dq_t<E, DQK, DV, 2>(p, s);
    case 3: return bwd_dq_t<E, DQK, DV, 3>(p, s);
    default:
      if constexpr (std::is_same<E, bf16>::value) {
        switch (mask_mode(p, causal)) {
          case 4: return bwd_dq_t<E, DQK, DV, 4>(p, s);
          case 5: return bwd_dq_t<E, DQK, DV, 5>(p, s);
          case 6: return bwd_dq_t<E, DQK, DV, 6>(p, s);
          case 7: return bwd_dq_t<E, DQK, DV, 7>(p, s);
          case 8: return bwd_dq_t<E, DQK, DV, 8>(p, s);
          default: return bwd_dq_t<E, DQK, DV, 9>(p, s);
        }
      } else {
        return hipErrorInvalidValue;
      }
  }
}

template <class E>
static hipError_t dq_t(const BwdParams& p, int d_qk, int d_v, bool causal, hipStream_t s) {
  if (d_qk == 64 && d_v == 64) return dq_m<E, 64, 64>(p, causal, s);
  if (d_qk == 128 && d_v == 128) return dq_m<E, 128, 128>(p, causal, s);
  if (d_qk == 192 && d_v == 128) return dq_m<E, 192, 128>(p, causal, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq(const BwdParams& p, ElemType et, int d_qk, int d_v, bool causal, hipStream_t s) {
  return et == ELEM_F16 ? dq_t<f16>(p, d_qk, d_v, causal, s) : dq_t<bf16>(p, d_qk, d_v, causal, s);
}

// Dense or padded batches (the two bodies walk the planner's work lists, whose sizes are
// those of the separate launches).
bool kvdq_merge_ok(const BwdParams& p, int d_qk, int d_v, bool causal) {
  return d_qk == 64 && d_v == 64 && mask_mode(p, causal) <= 1 && kvdq64_nkv(p) % 8 == 0;
}

hipError_t launch_bwd_kvdq(const BwdParams& p, ElemType et, bool causal, hipStream_t s) {
  if (et == ELEM_F16) return causal ? bwd_kvdq64_t<f16, 1>(p, s) : bwd_kvdq64_t<f16, 0>(p, s);
  return causal ? bwd_kvdq64_t<bf16, 1>(p, s) : bwd_kvdq64_t<bf16, 0>(p, s);
}

int dq_block_rows(int d_qk) {
  return d_qk == 64 ? DqShape<64>::BM : d_qk == 128 ? DqShape<128>::BM : DqShape<192>::BM;
}

template <class E>
static hipError_t finalize_t(const BwdParams& p, int d_qk, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.NH * p.Tpad;
  if (d_qk == 64)
    hipLaunchKernelGGL((bwd_finalize_kernel<E, 64>), dim3(blocks_for(rows * 8)), dim3(256), 0, s, p);
  else if (d_qk == 128)
    hipLaunchKernelGGL((bwd_finalize_kernel<E, 128>), dim3(blocks_for(rows * 16)), dim3(256), 0, s, p);
  else if (d_qk == 192)
    hipLaunchKernelGGL((bwd_finalize_kernel<E, 192>), dim3(blocks_for(rows * 24)), dim3(256), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_finalize(const BwdParams& p, ElemType et, int d_qk, hipStream_t s) {
  return et == ELEM_F16 ? finalize_t<f16>(p, d_qk, s) : finalize_t<bf16>(p, d_qk, s);
}

}  // namespace attn53
