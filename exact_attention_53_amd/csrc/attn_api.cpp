// C ABI of the attention library: argument validation, workspace layout and kernel
// dispatch.  No device memory is allocated here and no state is kept between calls.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/attn53.h"
#include "attn_kernels.hpp"

using attn53::BwdParams;
using attn53::FwdParams;
using attn53::kRowPad;
using attn53::Strides;

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool headdims_supported(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
}

attn_status check_sizes(int B, int NH, int T, int dqk, int dv) {
  if (B < 1 || NH < 1 || T < 1) return ATTN_ERR_SHAPE;
  const int64_t rows = (int64_t)B * NH * ((int64_t)T + kRowPad);
  if (rows > (int64_t)INT32_MAX) return ATTN_ERR_SHAPE;
  if (!headdims_supported(dqk, dv)) return ATTN_ERR_HEADDIM;
  return ATTN_OK;
}

struct Extent {
  uintptr_t lo, hi;  // byte range [lo, hi)
};

// Validates one bf16 (B, NH, T, d) tensor and returns its byte extent.
attn_status check_tensor(const void* ptr, attn_strides s, int B, int NH, int T, int d, Extent* ext) {
  if (ptr == nullptr) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return ATTN_ERR_ALIGN;
  if (s.b < 0 || s.h < 0 || s.t < 0 || s.b % 8 || s.h % 8 || s.t % 8) return ATTN_ERR_STRIDE;
  if (s.t > (int64_t)1 << 24) return ATTN_ERR_STRIDE;  // keeps per-tile byte offsets within 32 bits
  const int64_t last = s.b * (B - 1) + s.h * (NH - 1) + s.t * (int64_t)(T - 1) + d;
  ext->lo = reinterpret_cast<uintptr_t>(ptr);
  ext->hi = ext->lo + (uintptr_t)last * 2u;
  return ATTN_OK;
}

bool overlaps(const Extent& a, const Extent& b) { return a.lo < b.hi && b.lo < a.hi; }

Strides cvt(attn_strides s) { return Strides{s.b, s.h, s.t}; }

int64_t tpad(int T) { return ((int64_t)T + kRowPad - 1) / kRowPad * kRowPad; }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t ws_D_bytes(int B, int NH, int T) { return align256((size_t)B * NH * tpad(T) * 4); }

size_t ws_acc_bytes(int B, int NH, int T, int dqk) { return align256((size_t)B * NH * tpad(T) * dqk * 4); }

attn_status hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, NH and T must be >= 1 and B*NH*T must fit in int32";
    case ATTN_ERR_HEADDIM: return "unsupported head dims: (d_qk, d_v) must be (64,64), (128,128) or (192,128)";
    case ATTN_ERR_STRIDE: return "strides must be non-negative multiples of 8 elements, the t stride at most 2^24";
    case ATTN_ERR_ALIGN: return "tensor pointers must be 16-byte aligned";
    case ATTN_ERR_WORKSPACE: return "workspace is NULL, misaligned or smaller than attn_bwd_workspace_bytes()";
    case ATTN_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case ATTN_ERR_ARG: return "invalid argument: scale must be finite and > 0, flags 0 or 1, stage mask non-empty";
    case ATTN_ERR_ALIAS: return "an output tensor overlaps an input tensor";
  }
  return "unknown attn_status";
}

int attn_version(void) { return 100; }

attn_status attn_fwd(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                     attn_strides sv, void* o, attn_strides so, float* lse, int B, int NH, int T, int d_qk,
                     int d_v, float scale, int causal, void* stream) {
  attn_status st = check_sizes(B, NH, T, d_qk, d_v);
  if (st != ATTN_OK) return st;
  if (!std::isfinite(scale) || !(scale > 0.f) || (causal != 0 && causal != 1)) return ATTN_ERR_ARG;
  Extent eq, ek, ev, eo;
  if ((st = check_tensor(q, sq, B, NH, T, d_qk, &eq)) != ATTN_OK) return st;
  if ((st = check_tensor(k, sk, B, NH, T, d_qk, &ek)) != ATTN_OK) return st;
  if ((st = check_tensor(v, sv, B, NH, T, d_v, &ev)) != ATTN_OK) return st;
  if ((st = check_tensor(o, so, B, NH, T, d_v, &eo)) != ATTN_OK) return st;
  if (lse != nullptr && reinterpret_cast<uintptr_t>(lse) % 4 != 0) return ATTN_ERR_ALIGN;
  if (overlaps(eo, eq) || overlaps(eo, ek) || overlaps(eo, ev)) return ATTN_ERR_ALIAS;
  if (lse != nullptr) {
    Extent el{reinterpret_cast<uintptr_t>(lse), reinterpret_cast<uintptr_t>(lse) + (uintptr_t)B * NH * T * 4u};
    if (overlaps(el, eq) || overlaps(el, ek) || overlaps(el, ev) || overlaps(el, eo)) return ATTN_ERR_ALIAS;
  }
  FwdParams p{};
  p.q = q; p.sq = cvt(sq);
  p.k = k; p.sk = cvt(sk);
  p.v = v; p.sv = cvt(sv);
  p.o = o; p.so = cvt(so);
  p.lse = lse;
  p.B = B; p.NH = NH; p.T = T;
  p.scale_log2 = scale * kLog2e;
  return hip_status(attn53::launch_fwd(p, d_qk, d_v, causal != 0, (hipStream_t)stream));
}

size_t attn_bwd_workspace_bytes(int B, int NH, int T, int d_qk, int d_v, int deterministic) {
  if (check_sizes(B, NH, T, d_qk, d_v) != ATTN_OK) return 0;
  size_t n = 2 * ws_D_bytes(B, NH, T);  // D and LSE log2(e)
  if (!deterministic) n += ws_acc_bytes(B, NH, T, d_qk);
  return n;
}

attn_status attn_bwd_staged(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                            attn_strides sv, const void* o, attn_strides so, const float* lse, const void* do_,
                            attn_strides sdo, void* dq, attn_strides sdq, void* dk, attn_strides sdk, void* dv,
                            attn_strides sdv, int B, int NH, int T, int d_qk, int d_v, float scale, int causal,
                            int deterministic, void* workspace, size_t workspace_bytes, void* stream,
                            unsigned stages) {
  attn_status st = check_sizes(B, NH, T, d_qk, d_v);
  if (st != ATTN_OK) return st;
  if (!std::isfinite(scale) || !(scale > 0.f) || (causal != 0 && causal != 1) ||
      (deterministic != 0 && deterministic != 1))
    return ATTN_ERR_ARG;
  if (stages == 0 || (stages & ~ATTN_BWD_ALL) != 0) return ATTN_ERR_ARG;
  Extent eq, ek, ev, eo, edo, edq, edk, edv;
  if ((st = check_tensor(q, sq, B, NH, T, d_qk, &eq)) != ATTN_OK) return st;
  if ((st = check_tensor(k, sk, B, NH, T, d_qk, &ek)) != ATTN_OK) return st;
  if ((st = check_tensor(v, sv, B, NH, T, d_v, &ev)) != ATTN_OK) return st;
  if ((st = check_tensor(o, so, B, NH, T, d_v, &eo)) != ATTN_OK) return st;
  if ((st = check_tensor(do_, sdo, B, NH, T, d_v, &edo)) != ATTN_OK) return st;
  if ((st = check_tensor(dq, sdq, B, NH, T, d_qk, &edq)) != ATTN_OK) return st;
  if ((st = check_tensor(dk, sdk, B, NH, T, d_qk, &edk)) != ATTN_OK) return st;
  if ((st = check_tensor(dv, sdv, B, NH, T, d_v, &edv)) != ATTN_OK) return st;
  if (lse == nullptr) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return ATTN_ERR_ALIGN;
  const Extent el{reinterpret_cast<uintptr_t>(lse), reinterpret_cast<uintptr_t>(lse) + (uintptr_t)B * NH * T * 4u};
  const size_t need = attn_bwd_workspace_bytes(B, NH, T, d_qk, d_v, deterministic);
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 16 != 0 || workspace_bytes < need)
    return ATTN_ERR_WORKSPACE;
  const Extent ew{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
  const Extent ins[] = {eq, ek, ev, eo, edo, el};
  const Extent outs[] = {edq, edk, edv, ew};
  for (const Extent& a : outs)
    for (const Extent& b : ins)
      if (overlaps(a, b)) return ATTN_ERR_ALIAS;
  if (overlaps(ew, edq) || overlaps(ew, edk) || overlaps(ew, edv)) return ATTN_ERR_ALIAS;

  BwdParams p{};
  p.q = q; p.sq = cvt(sq);
  p.k = k; p.sk = cvt(sk);
  p.v = v; p.sv = cvt(sv);
  p.o = o; p.so = cvt(so);
  p.lse = lse;
  p.dO = do_; p.sdo = cvt(sdo);
  p.dq = dq; p.sdq = cvt(sdq);
  p.dk = dk; p.sdk = cvt(sdk);
  p.dv = dv; p.sdv = cvt(sdv);
  p.B = B; p.NH = NH; p.T = T; p.Tpad = (int)tpad(T);
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  p.D = static_cast<float*>(workspace);
  p.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws_D_bytes(B, NH, T));
  p.dq_acc = deterministic ? nullptr
                           : reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * ws_D_bytes(B, NH, T));
  const hipStream_t s = (hipStream_t)stream;
  if (stages & ATTN_BWD_PREPROCESS) {
    st = hip_status(attn53::launch_bwd_preprocess(p, d_qk, d_v, !deterministic, s));
    if (st != ATTN_OK) return st;
  }
  if (stages & ATTN_BWD_MAIN) {
    st = hip_status(attn53::launch_bwd_main(p, d_qk, d_v, causal != 0, deterministic != 0, s));
    if (st != ATTN_OK) return st;
  }
  if (stages & ATTN_BWD_DQ) {
    st = hip_status(deterministic ? attn53::launch_bwd_dq(p, d_qk, d_v, causal != 0, s)
                                  : attn53::launch_bwd_finalize(p, d_qk, s));
    if (st != ATTN_OK) return st;
  }
  return ATTN_OK;
}

attn_status attn_bwd(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v, attn_strides sv,
                     const void* o, attn_strides so, const float* lse, const void* do_, attn_strides sdo, void* dq,
                     attn_strides sdq, void* dk, attn_strides sdk, void* dv, attn_strides sdv, int B, int NH, int T,
                     int d_qk, int d_v, float scale, int causal, int deterministic, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return attn_bwd_staged(q, sq, k, sk, v, sv, o, so, lse, do_, sdo, dq, sdq, dk, sdk, dv, sdv, B, NH, T, d_qk, d_v,
                         scale, causal, deterministic, workspace, workspace_bytes, stream, ATTN_BWD_ALL);
}

}  // extern "C"
