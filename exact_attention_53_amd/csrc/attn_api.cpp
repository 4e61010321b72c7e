// C ABI of the attention library: argument validation, workspace layout and kernel
// dispatch.  No device memory is allocated here and no state is kept between calls.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

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

// An output tensor must give every (b, h, t) row its own d elements: otherwise concurrent
// workgroups write the same bytes.  Sufficient (and, for the layouts in use, necessary)
// condition: with the dimensions of size > 1 sorted by stride, each stride is at least the
// extent of everything inside it (d for the innermost).
attn_status check_output_rows(attn_strides s, int B, int NH, int T, int d) {
  struct Dim {
    int64_t stride, size;
  } dims[3] = {{s.b, B}, {s.h, NH}, {s.t, T}};
  for (int i = 1; i < 3; ++i)  // insertion sort by stride
    for (int j = i; j > 0 && dims[j].stride < dims[j - 1].stride; --j) {
      const Dim t = dims[j];
      dims[j] = dims[j - 1];
      dims[j - 1] = t;
    }
  int64_t inner = d;
  for (const Dim& x : dims) {
    if (x.size <= 1) continue;
    if (x.stride < inner) return ATTN_ERR_STRIDE;
    inner = x.stride * x.size;
  }
  return ATTN_OK;
}

Strides cvt(attn_strides s) { return Strides{s.b, s.h, s.t}; }

int64_t tpad(int T) { return ((int64_t)T + kRowPad - 1) / kRowPad * kRowPad; }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t ws_D_bytes(int B, int NH, int T) { return align256((size_t)B * NH * tpad(T) * 4); }

size_t ws_acc_bytes(int B, int NH, int T, int dqk) { return align256((size_t)B * NH * tpad(T) * dqk * 4); }

attn_status hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

attn53::ElemType elem_type(attn_dtype d) { return d == ATTN_DTYPE_F16 ? attn53::ELEM_F16 : attn53::ELEM_BF16; }

// Sliding window (0 = none; >= 1) and ALiBi bias (0 / 1): each needs the causal mask and a
// dense (unpadded) batch; they do not combine.
bool window_ok(int window, int alibi, int causal, const int32_t* seq_q, const int32_t* seq_k) {
  if (window < 0 || (alibi != 0 && alibi != 1) || (window > 0 && alibi)) return false;
  return (window == 0 && alibi == 0) || (causal == 1 && seq_q == nullptr && seq_k == nullptr);
}

// Work list of a padded-batch launch: one (b, block) pair of int32 per item.
size_t ws_list_bytes(int B, int T, int block) { return align256((size_t)B * ((T + block - 1) / block) * 8); }

constexpr int kFwdBlock = 128;  // query rows per forward workgroup
constexpr int kKvBlock = 128;   // keys per key/value workgroup

bool int_ptr_ok(const int32_t* p) { return p != nullptr && reinterpret_cast<uintptr_t>(p) % 4 == 0; }

// Block-sparse map of a call (map == nullptr: none).
struct BsArgs {
  const uint8_t* map;
  int64_t sb, sh;  // element (byte) strides along b and h; 0 broadcasts
};

int bs_nb(int T) { return (T + attn53::kBsBlock - 1) / attn53::kBsBlock; }

// One set of block-sparse lists: per item a slot of nb int32 indices, a count, and the
// sorted work list (two int32 per item).
size_t bs_lists_bytes(int64_t items, int nb) {
  return align256((size_t)items * nb * 4) + align256((size_t)items * 4) + align256((size_t)items * 8);
}

// Lays out one set of lists at ws, builds them on the device (bs_index_kernel, then the
// cost-sorted work list); returns the bytes used.
attn_status bs_build(const BsArgs& bs, int B, int NH, int T, int kind, int group, int causal, char* ws,
                     attn53::BsList* out, size_t* used, hipStream_t s) {
  const int nb = bs_nb(T);
  const int nblk = (nb + group - 1) / group;
  const int64_t items = (int64_t)B * NH * nblk;
  int* idx = reinterpret_cast<int*>(ws);
  int* cnt = reinterpret_cast<int*>(ws + align256((size_t)items * nb * 4));
  int* list = reinterpret_cast<int*>(ws + align256((size_t)items * nb * 4) + align256((size_t)items * 4));
  attn53::BsIndexParams ip{bs.map, bs.sb, bs.sh, idx, cnt, NH, B * NH, nb, nblk, group, kind, causal};
  if (attn53::launch_bs_index(ip, s) != hipSuccess) return ATTN_ERR_HIP;
  attn53::PlanParams pp{nullptr, nullptr, list, B * NH, T, attn53::kBsBlock * group, attn53::PLAN_Q, causal, cnt};
  if (attn53::launch_plan(pp, s) != hipSuccess) return ATTN_ERR_HIP;
  *out = attn53::BsList{list, idx, cnt, nb};
  *used = bs_lists_bytes(items, nb);
  return ATTN_OK;
}

// Key bias of a call (bias == nullptr: none): fp32, (B or 1, NH or 1, T) through element
// strides along b and h (0 broadcasts), contiguous along t; dbias (or nullptr) has the
// same strides.
struct KbArgs {
  const float* bias;
  int64_t sb, sh;
  float* dbias;
};

// Byte extent of a (B, NH, T) fp32 tensor with element strides sb, sh, 1.
Extent f32_extent(const void* ptr, int64_t sb, int64_t sh, int B, int NH, int T) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
  return Extent{lo, lo + (uintptr_t)(sb * (B - 1) + sh * (NH - 1) + T) * 4u};
}

attn_status check_kbias(const KbArgs& kb, int B, int NH, int T) {
  if (kb.bias == nullptr) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(kb.bias) % 4 != 0) return ATTN_ERR_ALIGN;
  if (kb.dbias != nullptr && reinterpret_cast<uintptr_t>(kb.dbias) % 4 != 0) return ATTN_ERR_ALIGN;
  if (kb.sb < 0 || kb.sh < 0) return ATTN_ERR_STRIDE;
  if (kb.dbias != nullptr) {  // distinct dbias rows must not share elements
    const int Bb = (B > 1 && kb.sb == 0) ? 1 : B, Hb = (NH > 1 && kb.sh == 0) ? 1 : NH;
    // rows (b, h) of T elements: the (b, h) strides as the outer dimensions of T-wide rows
    if (check_output_rows(attn_strides{0, kb.sb, kb.sh}, 1, Bb, Hb, T) != ATTN_OK) return ATTN_ERR_STRIDE;
  }
  return ATTN_OK;
}

size_t kb_ws_bytes(int B, int NH, int T) { return align256((size_t)B * NH * tpad(T) * 4); }

// Dropout of a call (mask == nullptr: none): the keep bits written by attn_dropout_mask.
struct DrArgs {
  const void* mask;
  float p;
};

int64_t drop_tp(int T) { return ((int64_t)T + 127) / 128 * 128; }

size_t drop_mask_bytes(int B, int NH, int T) {
  const int64_t tp = drop_tp(T);
  return (size_t)2 * B * NH * tp * (tp / 8);
}

attn_status check_dropout(const DrArgs& d, int B, int NH, int T, Extent* ext) {
  if (d.mask == nullptr) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(d.mask) % 16 != 0) return ATTN_ERR_ALIGN;
  if (!std::isfinite(d.p) || d.p < 0.f || d.p >= 1.f) return ATTN_ERR_ARG;
  ext->lo = reinterpret_cast<uintptr_t>(d.mask);
  ext->hi = ext->lo + drop_mask_bytes(B, NH, T);
  return ATTN_OK;
}

// Validates a block-sparse map and returns its byte extent.
attn_status check_map(const BsArgs& bs, int B, int NH, int T, Extent* ext) {
  if (bs.map == nullptr) return ATTN_ERR_NULL;
  if (bs.sb < 0 || bs.sh < 0) return ATTN_ERR_STRIDE;
  const int64_t nb = bs_nb(T);
  ext->lo = reinterpret_cast<uintptr_t>(bs.map);
  ext->hi = ext->lo + (uintptr_t)(bs.sb * (B - 1) + bs.sh * (NH - 1) + nb * nb);
  return ATTN_OK;
}

size_t fwd_bs_ws_bytes(int B, int NH, int T) { return bs_lists_bytes((int64_t)B * NH * bs_nb(T), bs_nb(T)); }

attn_status fwd_impl(attn53::ElemType et, const void* q, attn_strides sq, const void* k, attn_strides sk,
                     const void* v, attn_strides sv, void* o, attn_strides so, float* lse, const int32_t* seq_q,
                     const int32_t* seq_k, int B, int NH, int T, int d_qk, int d_v, float scale, int causal,
                     int window, int alibi, void* workspace, size_t workspace_bytes, void* stream,
                     const BsArgs* bs = nullptr, const KbArgs* kb = nullptr, const DrArgs* dr = nullptr) {
  attn_status st = check_sizes(B, NH, T, d_qk, d_v);
  if (st != ATTN_OK) return st;
  if (!std::isfinite(scale) || !(scale > 0.f) || (causal != 0 && causal != 1)) return ATTN_ERR_ARG;
  if (!window_ok(window, alibi, causal, seq_q, seq_k)) return ATTN_ERR_ARG;
  if ((bs != nullptr || kb != nullptr || dr != nullptr) &&
      (window != 0 || alibi != 0 || seq_q != nullptr || seq_k != nullptr || et != attn53::ELEM_BF16))
    return ATTN_ERR_ARG;
  if (kb != nullptr && (st = check_kbias(*kb, B, NH, T)) != ATTN_OK) return st;
  Extent edr{0, 0};
  if (dr != nullptr && (st = check_dropout(*dr, B, NH, T, &edr)) != ATTN_OK) return st;
  Extent eq, ek, ev, eo;
  if ((st = check_tensor(q, sq, B, NH, T, d_qk, &eq)) != ATTN_OK) return st;
  if ((st = check_tensor(k, sk, B, NH, T, d_qk, &ek)) != ATTN_OK) return st;
  if ((st = check_tensor(v, sv, B, NH, T, d_v, &ev)) != ATTN_OK) return st;
  if ((st = check_tensor(o, so, B, NH, T, d_v, &eo)) != ATTN_OK) return st;
  if ((st = check_output_rows(so, B, NH, T, d_v)) != ATTN_OK) return st;
  if (lse != nullptr && reinterpret_cast<uintptr_t>(lse) % 4 != 0) return ATTN_ERR_ALIGN;
  if (overlaps(eo, eq) || overlaps(eo, ek) || overlaps(eo, ev)) return ATTN_ERR_ALIAS;
  Extent el{0, 0};
  if (lse != nullptr) {
    el = Extent{reinterpret_cast<uintptr_t>(lse), reinterpret_cast<uintptr_t>(lse) + (uintptr_t)B * NH * T * 4u};
    if (overlaps(el, eq) || overlaps(el, ek) || overlaps(el, ev) || overlaps(el, eo)) return ATTN_ERR_ALIAS;
  }
  const bool varlen = seq_q != nullptr || seq_k != nullptr;
  if (dr != nullptr && (overlaps(eo, edr) || (lse != nullptr && overlaps(el, edr)))) return ATTN_ERR_ALIAS;
  Extent em{0, 0};
  if (bs != nullptr) {
    if ((st = check_map(*bs, B, NH, T, &em)) != ATTN_OK) return st;
    if (overlaps(eo, em) || (lse != nullptr && overlaps(el, em))) return ATTN_ERR_ALIAS;
  }
  if (kb != nullptr) {
    const Extent eb = f32_extent(kb->bias, kb->sb, kb->sh, B, NH, T);
    if (overlaps(eo, eb) || (lse != nullptr && overlaps(el, eb))) return ATTN_ERR_ALIAS;
    em = eb;  // the workspace must not overlap it either
  }
  if (varlen || bs != nullptr || kb != nullptr) {
    if (varlen && (seq_q == nullptr || seq_k == nullptr)) return ATTN_ERR_NULL;
    if (varlen && (!int_ptr_ok(seq_q) || !int_ptr_ok(seq_k))) return ATTN_ERR_ALIGN;
    const size_t need = varlen ? ws_list_bytes(B, T, kFwdBlock) : kb != nullptr ? kb_ws_bytes(B, NH, T)
                                                                                : fwd_bs_ws_bytes(B, NH, T);
    if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 16 != 0 || workspace_bytes < need)
      return ATTN_ERR_WORKSPACE;
    const Extent ew{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
    if (overlaps(ew, eq) || overlaps(ew, ek) || overlaps(ew, ev) || overlaps(ew, eo) ||
        (lse != nullptr && overlaps(ew, el)) || ((bs != nullptr || kb != nullptr) && overlaps(ew, em)))
      return ATTN_ERR_ALIAS;
  }
  FwdParams p{};
  p.q = q; p.sq = cvt(sq);
  p.k = k; p.sk = cvt(sk);
  p.v = v; p.sv = cvt(sv);
  p.o = o; p.so = cvt(so);
  p.lse = lse;
  p.B = B; p.NH = NH; p.T = T; p.Tk = T;
  p.scale_log2 = scale * kLog2e;
  p.win = window > 0 ? window : attn53::kNoWindow;
  p.alibi = alibi;
  const hipStream_t s = (hipStream_t)stream;
  if (varlen) {
    attn53::PlanParams pp{seq_q, seq_k, static_cast<int*>(workspace), B, T, kFwdBlock, attn53::PLAN_Q, causal};
    if ((st = hip_status(attn53::launch_plan(pp, s))) != ATTN_OK) return st;
    p.seq_q = seq_q;
    p.seq_k = seq_k;
    p.items = static_cast<const int*>(workspace);
  }
  if (bs != nullptr) {
    size_t used = 0;
    if ((st = bs_build(*bs, B, NH, T, 0, 1, causal, static_cast<char*>(workspace), &p.bs, &used, s)) != ATTN_OK)
      return st;
  }
  if (kb != nullptr) {
    float* kbs = static_cast<float*>(workspace);
    if ((st = hip_status(attn53::launch_bias_prep(kb->bias, kb->sb, kb->sh, 1.f / scale, kbs, (int)tpad(T), B, NH, T,
                                                  s))) != ATTN_OK)
      return st;
    p.kbias = kbs;
    p.kbias_ld = (int)tpad(T);
  }
  if (dr != nullptr) {
    p.drop_rows = static_cast<const unsigned char*>(dr->mask);
    p.drop_ld = (int)(drop_tp(T) / 8);
    p.drop_scale = 1.f / (1.f - dr->p);
  }
  return hip_status(attn53::launch_fwd(p, et, d_qk, d_v, causal != 0, s));
}

size_t bwd_ws_bytes(int B, int NH, int T, int d_qk, int d_v, int deterministic, bool varlen, bool bsp = false,
                    bool kbias = false) {
  if (check_sizes(B, NH, T, d_qk, d_v) != ATTN_OK || (deterministic != 0 && deterministic != 1)) return 0;
  size_t n = 2 * ws_D_bytes(B, NH, T);  // D and LSE log2(e)
  if (!deterministic) n += ws_acc_bytes(B, NH, T, d_qk);
  if (varlen) n += ws_list_bytes(B, T, kKvBlock) + ws_list_bytes(B, T, attn53::dq_block_rows(d_qk));
  if (bsp) {  // key-block columns, then groups of dQ query-block rows
    const int nb = bs_nb(T), group = attn53::dq_block_rows(d_qk) / attn53::kBsBlock;
    n += bs_lists_bytes((int64_t)B * NH * nb, nb) + bs_lists_bytes((int64_t)B * NH * ((nb + group - 1) / group), nb);
  }
  if (kbias) n += 2 * kb_ws_bytes(B, NH, T);  // the bias in score units; the per-head dbias sums
  return n;
}

attn_status bwd_impl(attn53::ElemType et, const void* q, attn_strides sq, const void* k, attn_strides sk,
                     const void* v, attn_strides sv, const void* o, attn_strides so, const float* lse,
                     const void* do_, attn_strides sdo, void* dq, attn_strides sdq, void* dk, attn_strides sdk,
                     void* dv, attn_strides sdv, const int32_t* seq_q, const int32_t* seq_k, int B, int NH, int T,
                     int d_qk, int d_v, float scale, int causal, int window, int alibi, int deterministic,
                     void* workspace, size_t workspace_bytes, void* stream, unsigned stages,
                     const BsArgs* bs = nullptr, const KbArgs* kb = nullptr, const DrArgs* dr = nullptr) {
  attn_status st = check_sizes(B, NH, T, d_qk, d_v);
  if (st != ATTN_OK) return st;
  if (!std::isfinite(scale) || !(scale > 0.f) || (causal != 0 && causal != 1) ||
      (deterministic != 0 && deterministic != 1))
    return ATTN_ERR_ARG;
  if (!window_ok(window, alibi, causal, seq_q, seq_k)) return ATTN_ERR_ARG;
  if ((bs != nullptr || kb != nullptr || dr != nullptr) &&
      (window != 0 || alibi != 0 || seq_q != nullptr || seq_k != nullptr || et != attn53::ELEM_BF16))
    return ATTN_ERR_ARG;
  if (kb != nullptr && (st = check_kbias(*kb, B, NH, T)) != ATTN_OK) return st;
  Extent edr{0, 0};
  if (dr != nullptr && (st = check_dropout(*dr, B, NH, T, &edr)) != ATTN_OK) return st;
  if (stages == 0 || (stages & ~ATTN_BWD_ALL) != 0) return ATTN_ERR_ARG;
  const bool varlen = seq_q != nullptr || seq_k != nullptr;
  if (varlen) {
    if (seq_q == nullptr || seq_k == nullptr) return ATTN_ERR_NULL;
    if (!int_ptr_ok(seq_q) || !int_ptr_ok(seq_k)) return ATTN_ERR_ALIGN;
  }
  Extent eq, ek, ev, eo, edo, edq, edk, edv;
  if ((st = check_tensor(q, sq, B, NH, T, d_qk, &eq)) != ATTN_OK) return st;
  if ((st = check_tensor(k, sk, B, NH, T, d_qk, &ek)) != ATTN_OK) return st;
  if ((st = check_tensor(v, sv, B, NH, T, d_v, &ev)) != ATTN_OK) return st;
  if ((st = check_tensor(o, so, B, NH, T, d_v, &eo)) != ATTN_OK) return st;
  if ((st = check_tensor(do_, sdo, B, NH, T, d_v, &edo)) != ATTN_OK) return st;
  if ((st = check_tensor(dq, sdq, B, NH, T, d_qk, &edq)) != ATTN_OK) return st;
  if ((st = check_tensor(dk, sdk, B, NH, T, d_qk, &edk)) != ATTN_OK) return st;
  if ((st = check_tensor(dv, sdv, B, NH, T, d_v, &edv)) != ATTN_OK) return st;
  if ((st = check_output_rows(sdq, B, NH, T, d_qk)) != ATTN_OK) return st;
  if ((st = check_output_rows(sdk, B, NH, T, d_qk)) != ATTN_OK) return st;
  if ((st = check_output_rows(sdv, B, NH, T, d_v)) != ATTN_OK) return st;
  if (lse == nullptr) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return ATTN_ERR_ALIGN;
  const Extent el{reinterpret_cast<uintptr_t>(lse), reinterpret_cast<uintptr_t>(lse) + (uintptr_t)B * NH * T * 4u};
  Extent em{0, 0};
  if (bs != nullptr && (st = check_map(*bs, B, NH, T, &em)) != ATTN_OK) return st;
  if (kb != nullptr) em = f32_extent(kb->bias, kb->sb, kb->sh, B, NH, T);
  if (dr != nullptr) em = edr;  // the mask is an input like the others
  const size_t need = bwd_ws_bytes(B, NH, T, d_qk, d_v, deterministic, varlen, bs != nullptr, kb != nullptr);
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 16 != 0 || workspace_bytes < need)
    return ATTN_ERR_WORKSPACE;
  const Extent ew{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
  const Extent ins[] = {eq, ek, ev, eo, edo, el, em};
  const Extent outs[] = {edq, edk, edv, ew};
  for (const Extent& a : outs)
    for (const Extent& b : ins)
      if (overlaps(a, b)) return ATTN_ERR_ALIAS;
  if (overlaps(ew, edq) || overlaps(ew, edk) || overlaps(ew, edv)) return ATTN_ERR_ALIAS;
  if (kb != nullptr && kb->dbias != nullptr) {
    const Extent edb = f32_extent(kb->dbias, kb->sb, kb->sh, B, NH, T);
    for (const Extent& a : ins)
      if (overlaps(edb, a)) return ATTN_ERR_ALIAS;
    if (overlaps(edb, ew) || overlaps(edb, edq) || overlaps(edb, edk) || overlaps(edb, edv)) return ATTN_ERR_ALIAS;
  }

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
  p.win = window > 0 ? window : attn53::kNoWindow;
  p.alibi = alibi;
  char* ws = static_cast<char*>(workspace);
  p.D = reinterpret_cast<float*>(ws);
  p.lse2 = reinterpret_cast<float*>(ws + ws_D_bytes(B, NH, T));
  size_t off = 2 * ws_D_bytes(B, NH, T);
  if (!deterministic) {
    p.dq_acc = reinterpret_cast<float*>(ws + off);
    off += ws_acc_bytes(B, NH, T, d_qk);
  }
  const hipStream_t s = (hipStream_t)stream;
  if (varlen) {
    p.seq_q = seq_q;
    p.seq_k = seq_k;
    int* list_kv = reinterpret_cast<int*>(ws + off);
    int* list_dq = reinterpret_cast<int*>(ws + off + ws_list_bytes(B, T, kKvBlock));
    p.items_kv = list_kv;
    p.items_dq = list_dq;
    if (stages & ATTN_BWD_MAIN) {
      attn53::PlanParams pp{seq_q, seq_k, list_kv, B, T, kKvBlock, attn53::PLAN_KV, causal};
      if ((st = hip_status(attn53::launch_plan(pp, s))) != ATTN_OK) return st;
    }
    if ((stages & ATTN_BWD_DQ) && deterministic) {
      attn53::PlanParams pp{seq_q, seq_k, list_dq, B, T, attn53::dq_block_rows(d_qk), attn53::PLAN_Q, causal};
      if ((st = hip_status(attn53::launch_plan(pp, s))) != ATTN_OK) return st;
    }
  }
  if (bs != nullptr) {
    size_t used = 0;
    char* lists = ws + off;
    if (stages & ATTN_BWD_MAIN) {
      if ((st = bs_build(*bs, B, NH, T, 1, 1, causal, lists, &p.bs_kv, &used, s)) != ATTN_OK) return st;
    }
    const int group = attn53::dq_block_rows(d_qk) / attn53::kBsBlock;
    lists += bs_lists_bytes((int64_t)B * NH * bs_nb(T), bs_nb(T));
    if ((stages & ATTN_BWD_DQ) && deterministic) {
      if ((st = bs_build(*bs, B, NH, T, 2, group, causal, lists, &p.bs_dq, &used, s)) != ATTN_OK) return st;
    }
    p.bsp = 1;
  }
  if (dr != nullptr) {
    const int64_t tp = drop_tp(T);
    p.drop_rows = static_cast<const unsigned char*>(dr->mask);
    p.drop_cols = p.drop_rows + (int64_t)B * NH * tp * (tp / 8);
    p.drop_ld = (int)(tp / 8);
    p.drop_tp = (int)tp;
    p.drop_scale = 1.f / (1.f - dr->p);
  }
  if (kb != nullptr) {  // the bias in score units (read by both kernels), the per-head dbias sums
    float* kbs = reinterpret_cast<float*>(ws + off);
    p.kbias = kbs;
    p.dbias_part = kb->dbias != nullptr ? reinterpret_cast<float*>(ws + off + kb_ws_bytes(B, NH, T)) : nullptr;
    if (stages & (ATTN_BWD_MAIN | ATTN_BWD_DQ)) {
      st = hip_status(attn53::launch_bias_prep(kb->bias, kb->sb, kb->sh, 1.f / scale, kbs, p.Tpad, B, NH, T, s));
      if (st != ATTN_OK) return st;
    }
  }
  if (stages & ATTN_BWD_PREPROCESS) {
    st = hip_status(attn53::launch_bwd_preprocess(p, et, d_qk, d_v, !deterministic, s));
    if (st != ATTN_OK) return st;
  }
  if ((stages & ATTN_BWD_MAIN) && (stages & ATTN_BWD_DQ) && deterministic &&
      attn53::kvdq_merge_ok(p, d_qk, d_v, causal != 0)) {
    return hip_status(attn53::launch_bwd_kvdq(p, et, causal != 0, s));  // both stages in one launch
  }
  if (stages & ATTN_BWD_MAIN) {
    st = hip_status(attn53::launch_bwd_main(p, et, d_qk, d_v, causal != 0, deterministic != 0, s));
    if (st != ATTN_OK) return st;
    if (p.dbias_part != nullptr) {
      st = hip_status(attn53::launch_dbias_reduce(p.dbias_part, p.Tpad, kb->dbias, kb->sb, kb->sh, B, NH, T, s));
      if (st != ATTN_OK) return st;
    }
  }
  if (stages & ATTN_BWD_DQ) {
    st = hip_status(deterministic ? attn53::launch_bwd_dq(p, et, d_qk, d_v, causal != 0, s)
                                  : attn53::launch_bwd_finalize(p, et, d_qk, s));
    if (st != ATTN_OK) return st;
  }
  return ATTN_OK;
}

// ---------------------------------------------------------------------------------
// Library-owned scratch for attn_bwd_noalloc: one static device array per GPU, so that
// callers that cannot allocate (graph capture, allocation-free serving loops) can still
// run the backward.  Its address on each device is looked up once, with that device
// current, and used for every kernel argument; the array's name is never used as an
// address in host code.
// ---------------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
attn_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return ATTN_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_bwd_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

attn_status attn_bwd_noalloc(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                             attn_strides sv, const void* o, attn_strides so, const float* lse, const void* do_,
                             attn_strides sdo, void* dq, attn_strides sdq, void* dk, attn_strides sdk, void* dv,
                             attn_strides sdv, int B, int NH, int T, int d_qk, int d_v, float scale, int causal,
                             int deterministic, void* stream) {
  const size_t need = bwd_ws_bytes(B, NH, T, d_qk, d_v, deterministic, false);
  if (need > kScratchBytes) return ATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {  // need == 0: invalid sizes or flags, reported by bwd_impl below
    const attn_status st = scratch_for_current_device(&ws);
    if (st != ATTN_OK) return st;
  }
  return bwd_impl(attn53::ELEM_BF16, q, sq, k, sk, v, sv, o, so, lse, do_, sdo, dq, sdq, dk, sdk, dv, sdv, nullptr,
                  nullptr, B, NH, T, d_qk, d_v, scale, causal, 0, 0, deterministic, ws, kScratchBytes, stream,
                  ATTN_BWD_ALL);
}

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, NH and T must be >= 1 and B*NH*T must fit in int32";
    case ATTN_ERR_HEADDIM: return "unsupported head dims: (d_qk, d_v) must be (64,64), (128,128) or (192,128)";
    case ATTN_ERR_STRIDE: return "strides must be non-negative multiples of 8 elements, the t stride at most 2^24";
    case ATTN_ERR_ALIGN: return "tensor pointers must be 16-byte aligned";
    case ATTN_ERR_WORKSPACE:
      return "workspace is NULL, misaligned or smaller than attn_bwd_workspace_bytes() (attn_bwd_noalloc: the "
             "sizes need more than its fixed scratch)";
    case ATTN_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case ATTN_ERR_ARG:
      return "invalid argument: scale must be finite and > 0, flags 0 or 1, stage mask non-empty, dtype known";
    case ATTN_ERR_ALIAS: return "an output tensor overlaps an input tensor";
  }
  return "unknown attn_status";
}

int attn_version(void) { return 400; }

size_t attn_fwd_blocksparse_workspace_bytes(int B, int NH, int T, int d_qk, int d_v) {
  if (check_sizes(B, NH, T, d_qk, d_v) != ATTN_OK) return 0;
  return fwd_bs_ws_bytes(B, NH, T);
}

attn_status attn_fwd_blocksparse(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                                 attn_strides sv, void* o, attn_strides so, float* lse, const uint8_t* block_map,
                                 int64_t map_stride_b, int64_t map_stride_h, int B, int NH, int T, int d_qk,
                                 int d_v, float scale, int causal, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  const BsArgs bs{block_map, map_stride_b, map_stride_h};
  return fwd_impl(attn53::ELEM_BF16, q, sq, k, sk, v, sv, o, so, lse, nullptr, nullptr, B, NH, T, d_qk, d_v, scale,
                  causal, 0, 0, workspace, workspace_bytes, stream, &bs);
}

size_t attn_dropout_mask_bytes(int B, int NH, int T) {
  if (B < 1 || NH < 1 || T < 1 || (int64_t)B * NH * ((int64_t)T + kRowPad) > (int64_t)INT32_MAX) return 0;
  const int64_t tp = drop_tp(T);
  if ((int64_t)B * NH * (tp / 64) * (tp / 128) > (int64_t)INT32_MAX) return 0;  // the mask kernel's grid
  return drop_mask_bytes(B, NH, T);
}

attn_status attn_dropout_mask(float p_drop, uint64_t seed, uint32_t offset, int B, int NH, int T, int causal,
                              void* mask, size_t mask_bytes, void* stream) {
  const size_t need = attn_dropout_mask_bytes(B, NH, T);
  if (need == 0) return ATTN_ERR_SHAPE;
  if (!std::isfinite(p_drop) || p_drop < 0.f || p_drop >= 1.f || (causal != 0 && causal != 1)) return ATTN_ERR_ARG;
  if (mask == nullptr) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(mask) % 16 != 0) return ATTN_ERR_ALIGN;
  if (mask_bytes < need) return ATTN_ERR_WORKSPACE;
  attn53::DropoutMaskParams p{};
  p.mask = static_cast<unsigned char*>(mask);
  p.B = B; p.NH = NH; p.Tp = (int)drop_tp(T); p.causal = causal;
  p.offset = offset;
  p.key0 = (uint32_t)(seed & 0xFFFFFFFFu);
  p.key1 = (uint32_t)(seed >> 32);
  const double thr = std::floor((double)p_drop * 65536.0 + 0.5);
  p.threshold = (uint32_t)(thr > 65536.0 ? 65536.0 : thr);
  return hip_status(attn53::launch_dropout_mask(p, (hipStream_t)stream));
}

attn_status attn_fwd_dropout(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                             attn_strides sv, void* o, attn_strides so, float* lse, const void* mask, float p_drop,
                             int B, int NH, int T, int d_qk, int d_v, float scale, int causal, void* stream) {
  const DrArgs dr{mask, p_drop};
  return fwd_impl(attn53::ELEM_BF16, q, sq, k, sk, v, sv, o, so, lse, nullptr, nullptr, B, NH, T, d_qk, d_v, scale,
                  causal, 0, 0, nullptr, 0, stream, nullptr, nullptr, &dr);
}

attn_status attn_bwd_dropout(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                             attn_strides sv, const void* o, attn_strides so, const float* lse, const void* do_,
                             attn_strides sdo, void* dq, attn_strides sdq, void* dk, attn_strides sdk, void* dv,
                             attn_strides sdv, const void* mask, float p_drop, int B, int NH, int T, int d_qk,
                             int d_v, float scale, int causal, int deterministic, void* workspace,
                             size_t workspace_bytes, void* stream, unsigned stages) {
  const DrArgs dr{mask, p_drop};
  return bwd_impl(attn53::ELEM_BF16, q, sq, k, sk, v, sv, o, so, lse, do_, sdo, dq, sdq, dk, sdk, dv, sdv, nullptr,
                  nullptr, B, NH, T, d_qk, d_v, scale, causal, 0, 0, deterministic, workspace, workspace_bytes,
                  stream, stages, nullptr, nullptr, &dr);
}

size_t fp8_vt_ld(int T) { return ((size_t)T + 63) / 64 * 64; }

size_t attn_fwd_fp8_workspace_bytes(int B, int NH, int T, int d_qk, int d_v) {
  if (B < 1 || NH < 1 || T < 1 || (int64_t)B * NH * ((int64_t)T + kRowPad) > (int64_t)INT32_MAX) return 0;
  if (d_qk != d_v || (d_qk != 64 && d_qk != 128)) return 0;
  return align256((size_t)B * NH * d_v * fp8_vt_ld(T));
}

attn_status attn_fwd_fp8(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                         attn_strides sv, void* o, attn_strides so, float* lse, float descale_q, float descale_k,
                         float descale_v, int B, int NH, int T, int d_qk, int d_v, float scale, int causal,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 1 || NH < 1 || T < 1 || (int64_t)B * NH * ((int64_t)T + kRowPad) > (int64_t)INT32_MAX)
    return ATTN_ERR_SHAPE;
  if (d_qk != d_v || (d_qk != 64 && d_qk != 128)) return ATTN_ERR_HEADDIM;
  for (float x : {scale, descale_q, descale_k, descale_v})
    if (!std::isfinite(x) || !(x > 0.f)) return ATTN_ERR_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  // fp8 tensors: one byte per element; rows 16-byte aligned for the 128-bit loads
  Extent e8[3];
  const void* ptrs[3] = {q, k, v};
  const attn_strides strd[3] = {sq, sk, sv};
  for (int i = 0; i < 3; ++i) {
    const attn_strides x = strd[i];
    if (ptrs[i] == nullptr) return ATTN_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % 16 != 0) return ATTN_ERR_ALIGN;
    if (x.b < 0 || x.h < 0 || x.t < 0 || x.b % 16 || x.h % 16 || x.t % 16 || x.t > (int64_t)1 << 24)
      return ATTN_ERR_STRIDE;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(ptrs[i]);
    e8[i] = Extent{lo, lo + (uintptr_t)(x.b * (B - 1) + x.h * (NH - 1) + x.t * (int64_t)(T - 1) + d_qk)};
  }
  attn_status st;
  Extent eo;
  if ((st = check_tensor(o, so, B, NH, T, d_v, &eo)) != ATTN_OK) return st;
  if ((st = check_output_rows(so, B, NH, T, d_v)) != ATTN_OK) return st;
  if (lse != nullptr && reinterpret_cast<uintptr_t>(lse) % 4 != 0) return ATTN_ERR_ALIGN;
  const Extent el{reinterpret_cast<uintptr_t>(lse), reinterpret_cast<uintptr_t>(lse) + (uintptr_t)B * NH * T * 4u};
  const size_t need = attn_fwd_fp8_workspace_bytes(B, NH, T, d_qk, d_v);
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 16 != 0 || workspace_bytes < need)
    return ATTN_ERR_WORKSPACE;
  const Extent ew{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
  for (const Extent& a : e8) {
    if (overlaps(eo, a) || overlaps(ew, a) || (lse != nullptr && overlaps(el, a))) return ATTN_ERR_ALIAS;
  }
  if (overlaps(ew, eo) || (lse != nullptr && (overlaps(el, eo) || overlaps(el, ew)))) return ATTN_ERR_ALIAS;
  attn53::Fp8FwdParams p{};
  p.q = q; p.sq = cvt(sq);
  p.k = k; p.sk = cvt(sk);
  p.v = v; p.sv = cvt(sv);
  p.vt = workspace; p.vt_ld = (int)fp8_vt_ld(T);
  p.o = o; p.so = cvt(so);
  p.lse = lse;
  p.B = B; p.NH = NH; p.T = T;
  p.scale_log2 = scale * descale_q * descale_k * kLog2e;
  p.descale_v = descale_v;
  return hip_status(attn53::launch_fwd_fp8(p, d_qk, causal != 0, (hipStream_t)stream));
}

size_t attn_fwd_keybias_workspace_bytes(int B, int NH, int T, int d_qk, int d_v) {
  if (check_sizes(B, NH, T, d_qk, d_v) != ATTN_OK) return 0;
  return kb_ws_bytes(B, NH, T);
}

attn_status attn_fwd_keybias(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                             attn_strides sv, void* o, attn_strides so, float* lse, const float* bias,
                             int64_t bias_stride_b, int64_t bias_stride_h, int B, int NH, int T, int d_qk, int d_v,
                             float scale, int causal, void* workspace, size_t workspace_bytes, void* stream) {
  const KbArgs kb{bias, bias_stride_b, bias_stride_h, nullptr};
  return fwd_impl(attn53::ELEM_BF16, q, sq, k, sk, v, sv, o, so, lse, nullptr, nullptr, B, NH, T, d_qk, d_v, scale,
                  causal, 0, 0, workspace, workspace_bytes, stream, nullptr, &kb);
}

size_t attn_bwd_keybias_workspace_bytes(int B, int NH, int T, int d_qk, int d_v, int deterministic) {
  return bwd_ws_bytes(B, NH, T, d_qk, d_v, deterministic, false, false, true);
}

attn_status attn_bwd_keybias(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                             attn_strides sv, const void* o, attn_strides so, const float* lse, const void* do_,
                             attn_strides sdo, void* dq, attn_strides sdq, void* dk, attn_strides sdk, void* dv,
                             attn_strides sdv, const float* bias, float* dbias, int64_t bias_stride_b,
                             int64_t bias_stride_h, int B, int NH, int T, int d_qk, int d_v, float scale, int causal,
                             int deterministic, void* workspace, size_t workspace_bytes, void* stream,
                             unsigned stages) {
  const KbArgs kb{bias, bias_stride_b, bias_stride_h, dbias};
  return bwd_impl(attn53::ELEM_BF16, q, sq, k, sk, v, sv, o, so, lse, do_, sdo, dq, sdq, dk, sdk, dv, sdv, nullptr,
                  nullptr, B, NH, T, d_qk, d_v, scale, causal, 0, 0, deterministic, workspace, workspace_bytes,
                  stream, stages, nullptr, &kb);
}

size_t attn_bwd_blocksparse_workspace_bytes(int B, int NH, int T, int d_qk, int d_v, int deterministic) {
  return bwd_ws_bytes(B, NH, T, d_qk, d_v, deterministic, false, true);
}

attn_status attn_bwd_blocksparse(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                                 attn_strides sv, const void* o, attn_strides so, const float* lse, const void* do_,
                                 attn_strides sdo, void* dq, attn_strides sdq, void* dk, attn_strides sdk, void* dv,
                                 attn_strides sdv, const uint8_t* block_map, int64_t map_stride_b,
                                 int64_t map_stride_h, int B, int NH, int T, int d_qk, int d_v, float scale,
                                 int causal, int deterministic, void* workspace, size_t workspace_bytes,
                                 void* stream, unsigned stages) {
  const BsArgs bs{block_map, map_stride_b, map_stride_h};
  return bwd_impl(attn53::ELEM_BF16, q, sq, k, sk, v, sv, o, so, lse, do_, sdo, dq, sdq, dk, sdk, dv, sdv, nullptr,
                  nullptr, B, NH, T, d_qk, d_v, scale, causal, 0, 0, deterministic, workspace, workspace_bytes,
                  stream, stages, &bs);
}

attn_status attn_fwd(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                     attn_strides sv, void* o, attn_strides so, float* lse, int B, int NH, int T, int d_qk,
                     int d_v, float scale, int causal, void* stream) {
  return fwd_impl(attn53::ELEM_BF16, q, sq, k, sk, v, sv, o, so, lse, nullptr, nullptr, B, NH, T, d_qk, d_v, scale, causal, 0, 0, nullptr, 0,
                  stream);
}

size_t attn_fwd_varlen_workspace_bytes(int B, int NH, int T, int d_qk, int d_v) {
  if (check_sizes(B, NH, T, d_qk, d_v) != ATTN_OK) return 0;
  return ws_list_bytes(B, T, kFwdBlock);
}

attn_status attn_fwd_varlen(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                            attn_strides sv, void* o, attn_strides so, float* lse, const int32_t* seq_len_q,
                            const int32_t* seq_len_kv, int B, int NH, int T, int d_qk, int d_v, float scale,
                            int causal, void* workspace, size_t workspace_bytes, void* stream) {
  if (seq_len_q == nullptr || seq_len_kv == nullptr) return ATTN_ERR_NULL;
  return fwd_impl(attn53::ELEM_BF16, q, sq, k, sk, v, sv, o, so, lse, seq_len_q, seq_len_kv, B, NH, T, d_qk, d_v, scale, causal,
                  0, 0, workspace, workspace_bytes, stream);
}

size_t attn_bwd_workspace_bytes(int B, int NH, int T, int d_qk, int d_v, int deterministic) {
  return bwd_ws_bytes(B, NH, T, d_qk, d_v, deterministic, false);
}

attn_status attn_bwd_staged(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                            attn_strides sv, const void* o, attn_strides so, const float* lse, const void* do_,
                            attn_strides sdo, void* dq, attn_strides sdq, void* dk, attn_strides sdk, void* dv,
                            attn_strides sdv, int B, int NH, int T, int d_qk, int d_v, float scale, int causal,
                            int deterministic, void* workspace, size_t workspace_bytes, void* stream,
                            unsigned stages) {
  return bwd_impl(attn53::ELEM_BF16, q, sq, k, sk, v, sv, o, so, lse, do_, sdo, dq, sdq, dk, sdk, dv, sdv, nullptr, nullptr, B, NH, T,
                  d_qk, d_v, scale, causal, 0, 0, deterministic, workspace, workspace_bytes, stream, stages);
}

attn_status attn_bwd(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v, attn_strides sv,
                     const void* o, attn_strides so, const float* lse, const void* do_, attn_strides sdo, void* dq,
                     attn_strides sdq, void* dk, attn_strides sdk, void* dv, attn_strides sdv, int B, int NH, int T,
                     int d_qk, int d_v, float scale, int causal, int deterministic, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return bwd_impl(attn53::ELEM_BF16, q, sq, k, sk, v, sv, o, so, lse, do_, sdo, dq, sdq, dk, sdk, dv, sdv, nullptr, nullptr, B, NH, T,
                  d_qk, d_v, scale, causal, 0, 0, deterministic, workspace, workspace_bytes, stream, ATTN_BWD_ALL);
}

size_t attn_bwd_varlen_workspace_bytes(int B, int NH, int T, int d_qk, int d_v, int deterministic) {
  return bwd_ws_bytes(B, NH, T, d_qk, d_v, deterministic, true);
}

attn_status attn_bwd_varlen(const void* q, attn_strides sq, const void* k, attn_strides sk, const void* v,
                            attn_strides sv, const void* o, attn_strides so, const float* lse, const void* do_,
                            attn_strides sdo, void* dq, attn_strides sdq, void* dk, attn_strides sdk, void* dv,
                            attn_strides sdv, const int32_t* seq_len_q, const int32_t* seq_len_kv, int B, int NH,
                            int T, int d_qk, int d_v, float scale, int causal, int deterministic, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (seq_len_q == nullptr || seq_len_kv == nullptr) return ATTN_ERR_NULL;
  return bwd_impl(attn53::ELEM_BF16, q, sq, k, sk, v, sv, o, so, lse, do_, sdo, dq, sdq, dk, sdk, dv, sdv, seq_len_q, seq_len_kv, B, NH,
                  T, d_qk, d_v, scale, causal, 0, 0, deterministic, workspace, workspace_bytes, stream, ATTN_BWD_ALL);
}

// Key split of a decode step: enough workgroups for two per CU (512), chunks of at least
// 1024 keys, at most 64 splits.
void decode_split(int B, int NH, int Tq, int Tk, int* nsplit, int* chunk) {
  const int64_t nbase = (int64_t)((Tq + kFwdBlock - 1) / kFwdBlock) * B * NH;
  int64_t n = 1;
  if (nbase < 512) n = std::min<int64_t>((512 + nbase - 1) / nbase, (Tk + 1023) / 1024);
  n = std::max<int64_t>(1, std::min<int64_t>(n, 64));
  const int64_t c = ((Tk + n - 1) / n + 63) / 64 * 64;
  *chunk = (int)c;
  *nsplit = (int)((Tk + c - 1) / c);
}

size_t decode_ws_bytes(int B, int NH, int Tq, int Tk, int d_v) {
  int n, c;
  decode_split(B, NH, Tq, Tk, &n, &c);
  return n > 1 ? align256((size_t)n * B * NH * Tq * (d_v + 1) * 4) : 0;
}

size_t attn_fwd_decode_workspace_bytes(int B, int NH, int Tq, int Tk, int d_qk, int d_v) {
  if (check_sizes(B, NH, Tq, d_qk, d_v) != ATTN_OK || check_sizes(B, NH, Tk, d_qk, d_v) != ATTN_OK) return 0;
  return decode_ws_bytes(B, NH, Tq, Tk, d_v);
}

attn_status attn_fwd_decode(attn_dtype dtype, const void* q, attn_strides sq, const void* k, attn_strides sk,
                            const void* v, attn_strides sv, void* o, attn_strides so, float* lse,
                            const int32_t* seq_len_kv, int B, int NH, int Tq, int Tk, int d_qk, int d_v,
                            float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16) return ATTN_ERR_ARG;
  attn_status st = check_sizes(B, NH, Tq, d_qk, d_v);
  if (st != ATTN_OK) return st;
  if ((st = check_sizes(B, NH, Tk, d_qk, d_v)) != ATTN_OK) return st;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_ARG;
  Extent eq, ek, ev, eo;
  if ((st = check_tensor(q, sq, B, NH, Tq, d_qk, &eq)) != ATTN_OK) return st;
  if ((st = check_tensor(k, sk, B, NH, Tk, d_qk, &ek)) != ATTN_OK) return st;
  if ((st = check_tensor(v, sv, B, NH, Tk, d_v, &ev)) != ATTN_OK) return st;
  if ((st = check_tensor(o, so, B, NH, Tq, d_v, &eo)) != ATTN_OK) return st;
  if ((st = check_output_rows(so, B, NH, Tq, d_v)) != ATTN_OK) return st;
  if (lse != nullptr && reinterpret_cast<uintptr_t>(lse) % 4 != 0) return ATTN_ERR_ALIGN;
  if (seq_len_kv != nullptr && !int_ptr_ok(seq_len_kv)) return ATTN_ERR_ALIGN;
  if (overlaps(eo, eq) || overlaps(eo, ek) || overlaps(eo, ev)) return ATTN_ERR_ALIAS;
  if (lse != nullptr) {
    const Extent el{reinterpret_cast<uintptr_t>(lse), reinterpret_cast<uintptr_t>(lse) + (uintptr_t)B * NH * Tq * 4u};
    if (overlaps(el, eq) || overlaps(el, ek) || overlaps(el, ev) || overlaps(el, eo)) return ATTN_ERR_ALIAS;
  }
  FwdParams p{};
  p.q = q; p.sq = cvt(sq);
  p.k = k; p.sk = cvt(sk);
  p.v = v; p.sv = cvt(sv);
  p.o = o; p.so = cvt(so);
  p.lse = lse;
  p.B = B; p.NH = NH; p.T = Tq; p.Tk = Tk;
  p.scale_log2 = scale * kLog2e;
  p.win = attn53::kNoWindow;
  p.seq_k = seq_len_kv;  // with items == nullptr: per-sequence key lengths only
  int nsplit, chunk;
  decode_split(B, NH, Tq, Tk, &nsplit, &chunk);
  if (nsplit == 1) return hip_status(attn53::launch_fwd(p, elem_type(dtype), d_qk, d_v, false, (hipStream_t)stream));
  const size_t need = decode_ws_bytes(B, NH, Tq, Tk, d_v);
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 16 != 0 || workspace_bytes < need)
    return ATTN_ERR_WORKSPACE;
  const Extent ew{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
  if (overlaps(ew, eq) || overlaps(ew, ek) || overlaps(ew, ev) || overlaps(ew, eo)) return ATTN_ERR_ALIAS;
  p.nsplit = nsplit;
  p.kv_chunk = chunk;
  p.part = static_cast<float*>(workspace);
  return hip_status(attn53::launch_fwd_split(p, elem_type(dtype), d_qk, d_v, (hipStream_t)stream));
}

attn_status attn_fwd_typed(attn_dtype dtype, const void* q, attn_strides sq, const void* k, attn_strides sk,
                           const void* v, attn_strides sv, void* o, attn_strides so, float* lse,
                           const int32_t* seq_len_q, const int32_t* seq_len_kv, int B, int NH, int T, int d_qk,
                           int d_v, float scale, int causal, int window, int alibi, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16) return ATTN_ERR_ARG;
  return fwd_impl(elem_type(dtype), q, sq, k, sk, v, sv, o, so, lse, seq_len_q, seq_len_kv, B, NH, T, d_qk, d_v,
                  scale, causal, window, alibi, workspace, workspace_bytes, stream);
}

attn_status attn_bwd_typed(attn_dtype dtype, const void* q, attn_strides sq, const void* k, attn_strides sk,
                           const void* v, attn_strides sv, const void* o, attn_strides so, const float* lse,
                           const void* do_, attn_strides sdo, void* dq, attn_strides sdq, void* dk, attn_strides sdk,
                           void* dv, attn_strides sdv, const int32_t* seq_len_q, const int32_t* seq_len_kv, int B,
                           int NH, int T, int d_qk, int d_v, float scale, int causal, int window, int alibi,
                           int deterministic, void* workspace, size_t workspace_bytes, void* stream,
                           unsigned stages) {
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16) return ATTN_ERR_ARG;
  return bwd_impl(elem_type(dtype), q, sq, k, sk, v, sv, o, so, lse, do_, sdo, dq, sdq, dk, sdk, dv, sdv, seq_len_q,
                  seq_len_kv, B, NH, T, d_qk, d_v, scale, causal, window, alibi, deterministic, workspace,
                  workspace_bytes, stream, stages);
}

}  // extern "C"
