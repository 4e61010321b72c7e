// Exact attention backward for gfx950: launchers of the preprocess and finalize
// kernels and dispatch of the per-configuration key/value and dQ launchers.  The
// kernels themselves are in attn_bwd_kernels.hpp.
#include "attn_bwd_kernels.hpp"

namespace attn53 {

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

hipError_t launch_bwd_main(const BwdParams& p, int d_qk, int d_v, bool causal, bool deterministic, hipStream_t s) {
  if (d_qk == 64 && d_v == 64)
    return causal ? bwd_main_t<64, 64, true>(p, deterministic, s) : bwd_main_t<64, 64, false>(p, deterministic, s);
  if (d_qk == 128 && d_v == 128)
    return causal ? bwd_main_t<128, 128, true>(p, deterministic, s) : bwd_main_t<128, 128, false>(p, deterministic, s);
  if (d_qk == 192 && d_v == 128)
    return causal ? bwd_main_t<192, 128, true>(p, deterministic, s) : bwd_main_t<192, 128, false>(p, deterministic, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq(const BwdParams& p, int d_qk, int d_v, bool causal, hipStream_t s) {
  if (d_qk == 64 && d_v == 64) return causal ? bwd_dq_t<64, 64, true>(p, s) : bwd_dq_t<64, 64, false>(p, s);
  if (d_qk == 128 && d_v == 128) return causal ? bwd_dq_t<128, 128, true>(p, s) : bwd_dq_t<128, 128, false>(p, s);
  if (d_qk == 192 && d_v == 128) return causal ? bwd_dq_t<192, 128, true>(p, s) : bwd_dq_t<192, 128, false>(p, s);
  return hipErrorInvalidValue;
}

int dq_block_rows(int d_qk) {
  return d_qk == 64 ? DqShape<64>::BM : d_qk == 128 ? DqShape<128>::BM : DqShape<192>::BM;
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
