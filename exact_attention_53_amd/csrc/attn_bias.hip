// Key bias: the per-key additive bias on the scores (the `bias` option among the SDPA
// options of [SA8 1.2], read as a bias over the keys, broadcast over the queries), and
// the reduction of its gradient.
//
// Pages cited (by title and section):
//   [SA8]  "ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析" 1.2 (bias option),
//          2.1 (dS, the gradient of the scores)
//
// bias_prep_kernel   copies the caller's bias, (B or 1, NH or 1, T) through element
//                    strides, into one row of Tpad floats per (b, h), divided by the scale:
//                    the kernels add it to the unscaled scores S = Q K^T, which are scaled
//                    afterwards.  Rows are zero past T.
// dbias_reduce_kernel dbias_j = sum_i dS_ij: the key/value kernel leaves that sum per
//                    (b, h, j); this kernel adds, for each element of the caller's dbias,
//                    the (b, h) pairs that share it (all batches where the bias has one row
//                    for every batch, all heads where it has one for every head), in one
//                    fixed order, b outer and h inner, so the result is bit-stable.
#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn53 {

__global__ __launch_bounds__(256) void bias_prep_kernel(const float* bias, int64_t sb, int64_t sh, float inv_scale,
                                                        float* out, int ld, int B, int NH, int T) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)B * NH * ld) return;
  const int t = (int)(i % ld);
  const int bh = (int)(i / ld);
  const int b = bh / NH, h = bh % NH;
  out[i] = t < T ? bias[b * sb + h * sh + t] * inv_scale : 0.f;
}

__global__ __launch_bounds__(256) void dbias_reduce_kernel(const float* part, int ld, float* dbias, int64_t sb,
                                                           int64_t sh, int B, int NH, int T) {
  // one thread per element (b', h', t) of the caller's bias shape
  const int Bb = (B > 1 && sb == 0) ? 1 : B, Hb = (NH > 1 && sh == 0) ? 1 : NH;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)Bb * Hb * T) return;
  const int t = (int)(i % T);
  const int bhb = (int)(i / T);
  const int b1 = bhb / Hb, h1 = bhb % Hb;
  float acc = 0.f;
  for (int b = (Bb == 1 ? 0 : b1); b < (Bb == 1 ? B : b1 + 1); ++b)
    for (int h = (Hb == 1 ? 0 : h1); h < (Hb == 1 ? NH : h1 + 1); ++h) acc += part[(int64_t)(b * NH + h) * ld + t];
  dbias[b1 * sb + h1 * sh + t] = acc;
}

hipError_t launch_bias_prep(const float* bias, int64_t sb, int64_t sh, float inv_scale, float* out, int ld, int B,
                            int NH, int T, hipStream_t s) {
  const int64_t n = (int64_t)B * NH * ld;
  hipLaunchKernelGGL(bias_prep_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, bias, sb, sh, inv_scale,
                     out, ld, B, NH, T);
  return hipGetLastError();
}

hipError_t launch_dbias_reduce(const float* part, int ld, float* dbias, int64_t sb, int64_t sh, int B, int NH, int T,
                               hipStream_t s) {
  const int Bb = (B > 1 && sb == 0) ? 1 : B, Hb = (NH > 1 && sh == 0) ? 1 : NH;
  const int64_t n = (int64_t)Bb * Hb * T;
  hipLaunchKernelGGL(dbias_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, ld, dbias, sb, sh,
                     B, NH, T);
  return hipGetLastError();
}

}  // namespace attn53
