// Kernel parameter blocks and launcher declarations (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn53 {

struct Strides {
  int64_t b, h, t;
};

struct FwdParams {
  const void* q; Strides sq;
  const void* k; Strides sk;
  const void* v; Strides sv;
  void* o; Strides so;
  float* lse;              // (B, NH, T) or nullptr
  int B, NH, T;
  float scale_log2;        // scale * log2(e)
};

struct BwdParams {
  const void* q; Strides sq;
  const void* k; Strides sk;
  const void* v; Strides sv;
  const void* o; Strides so;
  const float* lse;        // (B, NH, T)
  const void* dO; Strides sdo;
  void* dq; Strides sdq;
  void* dk; Strides sdk;
  void* dv; Strides sdv;
  int B, NH, T, Tpad;      // Tpad = T rounded up to kRowPad
  float scale;
  float scale_log2;
  float* D;                // workspace: (B, NH, Tpad) fp32, rowsum(dO * O)
  float* lse2;             // workspace: (B, NH, Tpad) fp32, LSE * log2(e) (+inf on padding)
  float* dq_acc;           // workspace: (B, NH, Tpad, d_qk) fp32, atomic mode only
};

constexpr int kRowPad = 128;

// Launchers: return hipSuccess or the launch error.  d_qk/d_v already validated.
hipError_t launch_fwd(const FwdParams& p, int d_qk, int d_v, bool causal, hipStream_t s);
hipError_t launch_bwd_preprocess(const BwdParams& p, int d_qk, int d_v, bool zero_acc, hipStream_t s);
hipError_t launch_bwd_main(const BwdParams& p, int d_qk, int d_v, bool causal, bool deterministic, hipStream_t s);
hipError_t launch_bwd_dq(const BwdParams& p, int d_qk, int d_v, bool causal, hipStream_t s);
hipError_t launch_bwd_finalize(const BwdParams& p, int d_qk, hipStream_t s);

}  // namespace attn53
