// Kernel parameter blocks and launcher declarations (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn53 {

struct Strides {
  int64_t b, h, t;
};

// Block-sparse map in the form the kernels walk (built on the device by bs_index_kernel
// from the caller's map, attn_blocksparse.hip).  For every work item (bh, blk) of a
// kernel, idx[(bh * nblk + blk) * nb ...] lists its live blocks of the other side in the
// order the kernel visits them and cnt[bh * nblk + blk] counts them; items[] is the work
// list (bh, blk) sorted by cost, longest first.  Blocks are kBsBlock x kBsBlock
// elements.  The dQ kernel's lists hold key block | (live query block rows of the
// item) << 16.  All nullptr: no block-sparse map.
struct BsList {
  const int* items;
  const int* idx;
  const int* cnt;
  int nb;                  // blocks along T: ceil(T / kBsBlock)
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
  BsList bs;               // block-sparse map: live key blocks per query block
  // Key bias (nullptr: none): kbias[(b * NH + h) * kbias_ld + j], the caller's bias of key j
  // divided by the scale (so that it adds to the unscaled scores), zero past T.
  const float* kbias;
  int kbias_ld;
  // Dropout (nullptr: none): query-major keep bits, drop_ld bytes per row, Tp rows per
  // head (attn_dropout.hip); kept weights are scaled by drop_scale = 1 / (1 - p).
  const unsigned char* drop_rows;
  int drop_ld;
  float drop_scale;
};

// Dropout keep masks (attn_dropout.hip): Tp = T rounded up to 128; mask holds the
// query-major bits (B * NH, Tp, Tp / 8 bytes), then the key-major bits of the same size.
struct DropoutMaskParams {
  unsigned char* mask;
  int B, NH, Tp, causal;
  uint32_t offset, key0, key1, threshold;
};

// Forward on fp8 (e4m3) inputs.  q, k, v hold e4m3 codes (strides in bytes); vt is the
// workspace's transposed copy of v, (B * NH, d, vt_ld) bytes with vt_ld = T rounded up to
// 64 (zero past T), written by the call's first kernel.
struct Fp8FwdParams {
  const void* q; Strides sq;
  const void* k; Strides sk;
  const void* v; Strides sv;
  void* vt; int vt_ld;
  void* o; Strides so;     // bf16
  float* lse;              // (B, NH, T) or nullptr
  int B, NH, T;
  float scale_log2;        // scale * descale_q * descale_k * log2(e)
  float descale_v;
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
  int bsp;                 // 1: block-sparse map (the lists below, built for the stages run)
  const float* kbias;      // key bias as in FwdParams, (B * NH, Tpad), or nullptr
  float* dbias_part;       // workspace: (B * NH, Tpad) fp32, sum over queries of dS per key
                           // (written by the key/value kernel when not nullptr)
  const unsigned char* drop_rows;  // dropout keep bits, query-major (nullptr: no dropout)
  const unsigned char* drop_cols;  // ... key-major
  int drop_ld, drop_tp;            // bytes per mask row; rows per head (T rounded up to 128)
  float drop_scale;                // 1 / (1 - p)
  BsList bs_kv;            // block-sparse map: live query blocks per key block (ascending)
  BsList bs_dq;            // ... live key blocks per dQ query block (descending, row bits)
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
  const int* counts;  // block-sparse: live blocks per item (B = B * NH items of T / block
                      // blocks); the cost is two 64-row tiles per live block
};

constexpr int kRowPad = 128;
constexpr int kBsBlock = 128;  // block-sparse map: elements per block along each side
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
// Deterministic mode, d = 64, plain or causal mask, dense or padded batches: the key/value
// and dQ kernels' work in one launch (kvdq_merge_ok says whether this configuration qualifies).
bool kvdq_merge_ok(const BwdParams& p, int d_qk, int d_v, bool causal);
hipError_t launch_bwd_kvdq(const BwdParams& p, ElemType et, bool causal, hipStream_t s);
hipError_t launch_bwd_finalize(const BwdParams& p, ElemType et, int d_qk, hipStream_t s);
hipError_t launch_plan(const PlanParams& p, hipStream_t s);
// fp8 forward (d_qk = d_v = d in {64, 128}): the transpose of v, then the forward kernel.
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, int d, bool causal, hipStream_t s);
// Block-sparse map -> per-item lists (see BsList).  kind: 0 query-block rows (forward,
// descending live key blocks, causal: up to the diagonal), 1 key-block columns (key/value
// kernel, ascending live query blocks, causal: from the diagonal), 2 groups of `group`
// query-block rows (dQ kernel, descending union of their live key blocks with row bits).
struct BsIndexParams {
  const unsigned char* map;
  int64_t msb, msh;        // element strides of the map along b and h (0: broadcast)
  int* idx;
  int* cnt;
  int NH, nbh, nb, nblk, group, kind, causal;
};
hipError_t launch_bs_index(const BsIndexParams& p, hipStream_t s);
// Key bias: the caller's bias (element strides sb, sh along b and h, 1 along t) divided by
// the scale into out (B * NH, ld) fp32, zero for t >= T; and the reduction of the per-head
// sums over queries of dS into the caller's dbias (same strides as the bias): each dbias
// element sums the (b, h) pairs that share it, b outer, h inner.
hipError_t launch_dropout_mask(const DropoutMaskParams& p, hipStream_t s);
hipError_t launch_bias_prep(const float* bias, int64_t sb, int64_t sh, float inv_scale, float* out, int ld, int B,
                            int NH, int T, hipStream_t s);
hipError_t launch_dbias_reduce(const float* part, int ld, float* dbias, int64_t sb, int64_t sh, int B, int NH, int T,
                               hipStream_t s);
// Query rows per workgroup of the dQ kernel (its work list uses blocks of this size).
int dq_block_rows(int d_qk);

}  // namespace attn53
