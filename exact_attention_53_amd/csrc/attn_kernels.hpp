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
  int B, NH, T;            // T: query rows (and key rows unless Tk says otherwise)
  int Tk;                  // key / value rows (decode: the cache length; otherwise T)
  // Key split (decode with few (b, h) pairs): workgroup id / nbase is the split; split c
  // covers keys [c kv_chunk, (c+1) kv_chunk) and writes its normalised fp32 partial O
  // (nsplit, B*NH, T, d_v) and LSE (nsplit, B*NH, T) to `part` for a merge kernel.
  int nsplit, kv_chunk;
  float* part;
  float scale_log2;        // scale * log2(e)
  int win;                 // causal sliding window: query i sees keys i-win+1 .. i
                           // (1 << 30 when there is no window)
  int alibi;               // 1: causal ALiBi bias -m_h (i - j), m_h = 2^(-8 (h+1) / NH)
  // Padded batches (all three set, or all nullptr): valid query / key rows per batch
  // (B int32 each; clamped to [0, T]) and the sorted work list of (b, query block).
  const int* seq_q;
  const int* seq_k;
  const int* items;
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
  int win;                 // causal sliding window as in FwdParams
  int alibi;               // ALiBi bias as in FwdParams
  float* D;                // workspace: (B, NH, Tpad) fp32, rowsum(dO * O)
  float* lse2;             // workspace: (B, NH, Tpad) fp32, LSE * log2(e) (+inf on padding)
  float* dq_acc;           // workspace: (B, NH, Tpad, d_qk) fp32, atomic mode only
  // Padded batches (all set, or all nullptr): valid query / key rows per batch and the
  // sorted work lists of the key/value kernel (b, key block) and the dQ kernel
  // (b, query block).
  const int* seq_q;
  const int* seq_k;
  const int* items_kv;
  const int* items_dq;
};

// Work lists of padded batches (see attn_plan.hip).  KIND_Q: query blocks of `block`
// rows, costed by the key tiles of 64 they visit; KIND_KV: key blocks of `block` keys,
// costed by the query steps of 64 rows they visit.
enum PlanKind { PLAN_Q = 0, PLAN_KV = 1 };
struct PlanParams {
  const int* seq_q;
  const int* seq_k;
  int* items;    // out: 2 int32 per item (b, block), longest first
  int B, T, block, kind, causal;
};

constexpr int kRowPad = 128;
constexpr int kNoWindow = 1 << 30;  // a window wider than any sequence

// 16-bit element type of Q, K, V, O, dO, dQ, dK, dV (one type per call).
enum ElemType { ELEM_BF16 = 0, ELEM_F16 = 1 };

// Launchers: return hipSuccess or the launch error.  d_qk/d_v already validated.
hipError_t launch_fwd(const FwdParams& p, ElemType et, int d_qk, int d_v, bool causal, hipStream_t s);
// Decode with a key split (p.nsplit > 1, non-causal): partial kernels, then the merge.
hipError_t launch_fwd_split(const FwdParams& p, ElemType et, int d_qk, int d_v, hipStream_t s);
hipError_t launch_bwd_preprocess(const BwdParams& p, ElemType et, int d_qk, int d_v, bool zero_acc, hipStream_t s);
hipError_t launch_bwd_main(const BwdParams& p, ElemType et, int d_qk, int d_v, bool causal, bool deterministic,
                           hipStream_t s);
hipError_t launch_bwd_dq(const BwdParams& p, ElemType et, int d_qk, int d_v, bool causal, hipStream_t s);
hipError_t launch_bwd_finalize(const BwdParams& p, ElemType et, int d_qk, hipStream_t s);
hipError_t launch_plan(const PlanParams& p, hipStream_t s);
// Query rows per workgroup of the dQ kernel (its work list uses blocks of this size).
int dq_block_rows(int d_qk);

}  // namespace attn53
