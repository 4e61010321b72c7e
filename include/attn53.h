/*
 * attn53.h — C ABI of a fused, tiled, exact scaled-dot-product attention library for
 * AMD Instinct MI355X (gfx950).  Forward and backward, bf16 or fp16 in/out, fp32 accumulation.
 *
 * Pages cited (by title and section):
 *   [SA8]  "ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析"
 *   [2CTA] "深度学习反向传播优化：2-CTA MMA模式与内存访问优化"
 *   [FAT]  "FlashAttention Triton实现中的内存访问模式优化与寄存器分配策略"
 *
 * Tensor conventions shared by every entry point
 * ---------------------------------------------
 *  - Q, K, V, O, dO, dQ, dK, dV are 16-bit tensors (bf16; fp16 through the entry points
 *    that take an attn_dtype) with logical shape (B, NH, T, d).
 *    Each is described by a device pointer plus an attn_strides value holding its
 *    element strides along b, h and t; the stride along d is always 1.  This covers
 *    the (B, T, NH, d) layout of the pages' output O, a (B, NH, T, d) layout, and the
 *    packed (B, T, 3, NH, HS) QKV block of [SA8 1.3]: with C = NH*HS, Q, K and V are
 *    base, base + C and base + 2C, each with strides {T*3*C, HS, 3*C}.  dQ, dK, dV may
 *    point into one packed buffer the same way.
 *  - Supported head widths (d_qk, d_v): (64, 64), (128, 128), (192, 128) — the head
 *    dims of the FA4 backward sweep [2CTA 4.1].  Anything else: ATTN_ERR_HEADDIM.
 *  - T_q == T_k == T >= 1, any value; partial tiles are masked inside the kernels.
 *  - Every tensor pointer must be 16-byte aligned and every stride a non-negative
 *    multiple of 8 elements, so that all global accesses are 128-bit; the t stride is
 *    at most 2^24 elements.  An output tensor (O, dQ, dK, dV) must also give each
 *    (b, h, t) row d elements of its own: with its dimensions of size > 1 sorted by
 *    stride, each stride is at least the extent of the dimensions inside it (d for the
 *    innermost).  Otherwise the call returns ATTN_ERR_ALIGN / ATTN_ERR_STRIDE.  There is
 *    no slow fallback.
 *  - LSE ("softmax stats" of [SA8 1.2, 1.3]) is fp32, contiguous (B, NH, T), and holds
 *    the natural-log logsumexp of each row of S = scale * Q K^T (mask applied).
 *  - causal = 1 masks key j > query i (top-left aligned, [SA8 2.2] loop bound).
 *  - scale multiplies Q K^T; the pages use 1/sqrt(d_k) [SA8 2.1].  Must be finite and
 *    > 0 (the kernels take each row maximum before scaling).
 *
 * Ownership, errors, execution
 * ----------------------------
 *  - The caller owns every buffer, including the backward workspace.  The library
 *    allocates no device memory and keeps no state between calls; calls are
 *    re-entrant and may run concurrently on different streams with distinct outputs.
 *  - Inputs are never written.  Outputs are overwritten (never accumulated into) and
 *    must not overlap any input's address range (ATTN_ERR_ALIAS).
 *  - Arguments are validated on the host before anything is launched; on error
 *    nothing is launched and nothing is written.  Launch failures report
 *    ATTN_ERR_HIP.  No C++ exception crosses this interface.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the legacy
 *    default stream).  Results are valid once the stream has been synchronised.
 */
#ifndef ATTN53_H
#define ATTN53_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,       /* a required pointer is NULL                         */
  ATTN_ERR_SHAPE = 2,      /* B, NH or T < 1, or the sizes overflow              */
  ATTN_ERR_HEADDIM = 3,    /* (d_qk, d_v) not one of the supported pairs          */
  ATTN_ERR_STRIDE = 4,     /* a stride negative, not a multiple of 8, t > 2^24,   */
                           /* or an output whose rows would share elements       */
  ATTN_ERR_ALIGN = 5,      /* a pointer is not 16-byte aligned                    */
  ATTN_ERR_WORKSPACE = 6,  /* workspace NULL or smaller than required             */
  ATTN_ERR_HIP = 7,        /* a HIP runtime call or kernel launch failed          */
  ATTN_ERR_ARG = 8,        /* scale not finite or <= 0, a flag not 0/1, bad stage mask */
  ATTN_ERR_ALIAS = 9       /* an output overlaps an input                         */
} attn_status;

/* Element strides of a (B, NH, T, d) view along b, h and t (the d stride is 1). */
typedef struct {
  int64_t b, h, t;
} attn_strides;

/* Human-readable text for a status code (static storage, never NULL). */
const char* attn_status_string(attn_status s);

/* Library version, major * 10000 + minor * 100 + patch. */
int attn_version(void);

/*
 * attn_fwd — exact attention forward [SA8 2.1 and A.1; FAT 2.2 and 4.2]:
 *   S = scale * Q K^T, causal mask, P = softmax(S) row-wise, O = P V,
 *   LSE_i = max_j S_ij + ln sum_j exp(S_ij - max_j S_ij).
 * One workgroup per query block keeps its Q tile on chip and streams K/V tiles with a
 * running max and running sum; O is normalised once at the end.
 *   q, k  : (B, NH, T, d_qk) bf16, strides sq, sk        (read)
 *   v     : (B, NH, T, d_v)  bf16, strides sv            (read)
 *   o     : (B, NH, T, d_v)  bf16, strides so            (written)
 *   lse   : (B, NH, T) fp32 contiguous, 4-byte aligned  (written), or NULL for
 *           inference, which skips the stats as the pages' inference mode does
 *           [SA8 1.2, 1.3].
 */
attn_status attn_fwd(const void* q, attn_strides sq,
                     const void* k, attn_strides sk,
                     const void* v, attn_strides sv,
                     void* o, attn_strides so,
                     float* lse,
                     int B, int NH, int T, int d_qk, int d_v,
                     float scale, int causal, void* stream);

/*
 * attn_bwd_workspace_bytes — device workspace that attn_bwd needs for these sizes.  The
 * cuDNN SDPA path of [SA8 1.3] asks the library for the size of the work memory a call
 * needs and hands it that much memory; here the caller queries this size and owns the
 * buffer (the library keeps no workspace of its own).  Holds D_i = sum_k dO_ik O_ik and
 * LSE_i log2(e) (fp32, one per row, rows padded to a multiple of 128) and, in atomic
 * mode, the fp32 dQ accumulator (B * NH * Tpad * d_qk fp32).  Pure function of its
 * arguments; launches nothing.  Returns 0 for invalid sizes or flags.
 */
size_t attn_bwd_workspace_bytes(int B, int NH, int T, int d_qk, int d_v, int deterministic);

/*
 * attn_bwd — exact attention backward [SA8 2.1 and A.2; 2CTA 2.2, 3.1, 3.2]:
 *   D   = rowsum(dO * O)            (equals (dP * P) 1 of [SA8 2.1 step 3])
 *   P   = exp(scale * Q K^T - LSE)  (recomputed from the forward's LSE)
 *   dV  = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
 *   dQ  = scale * dS K,  dK = scale * dS^T Q.
 * Workgroups own a key/value block, keep K, V and their dK, dV accumulators on chip
 * and loop over query blocks.  dQ needs a sum over key blocks [2CTA 2.2]:
 *   deterministic = 0: fp32 atomic adds into an fp32 accumulator in the workspace,
 *                      then one conversion pass to bf16 (run-to-run bits may differ);
 *   deterministic = 1: every dQ row block is summed over key blocks in one fixed
 *                      order inside a single workgroup, so all outputs are
 *                      bit-identical from run to run [2CTA 3.2].
 *   q, k, v, o, do_ : bf16 inputs as in attn_fwd (o is the forward's output)
 *   lse             : the forward's (B, NH, T) fp32 stats (read; must not be NULL)
 *   dq, dk, dv      : bf16 outputs (written), shapes of q, k, v
 *   workspace       : device memory of at least attn_bwd_workspace_bytes(...) bytes,
 *                     16-byte aligned, owned by the caller, clobbered by the call.
 */
attn_status attn_bwd(const void* q, attn_strides sq,
                     const void* k, attn_strides sk,
                     const void* v, attn_strides sv,
                     const void* o, attn_strides so,
                     const float* lse,
                     const void* do_, attn_strides sdo,
                     void* dq, attn_strides sdq,
                     void* dk, attn_strides sdk,
                     void* dv, attn_strides sdv,
                     int B, int NH, int T, int d_qk, int d_v,
                     float scale, int causal, int deterministic,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Stage bits for attn_bwd_staged; each stage is one kernel launch, except that with the
 * deterministic dQ at d_qk = d_v = 64 (plain or causal mask, dense or padded batches,
 * B * NH * ceil(T / 128) a multiple of 8) ATTN_BWD_MAIN and ATTN_BWD_DQ requested together
 * run as one launch, with results identical to the two launches. */
#define ATTN_BWD_PREPROCESS 1u /* D = rowsum(dO * O); atomic mode: clear the accumulator */
#define ATTN_BWD_MAIN 2u       /* key/value-stationary kernel: P recompute, dP, dS, dV,  */
                               /* dK; atomic mode also adds partial dQ sums atomically  */
#define ATTN_BWD_DQ 4u         /* atomic mode: dQ = scale * accumulator -> bf16;        */
                               /* deterministic mode: query-stationary dQ kernel        */
#define ATTN_BWD_ALL 7u

/*
 * attn_bwd_staged — attn_bwd restricted to the stages in `stages` (a non-empty subset
 * of ATTN_BWD_ALL).  Running the three stages one after another on one stream with the
 * same arguments and workspace is exactly attn_bwd.  Exists so that each stage's
 * kernels can be timed on their own; returns ATTN_ERR_ARG for an empty or unknown mask.
 */
attn_status attn_bwd_staged(const void* q, attn_strides sq,
                            const void* k, attn_strides sk,
                            const void* v, attn_strides sv,
                            const void* o, attn_strides so,
                            const float* lse,
                            const void* do_, attn_strides sdo,
                            void* dq, attn_strides sdq,
                            void* dk, attn_strides sdk,
                            void* dv, attn_strides sdv,
                            int B, int NH, int T, int d_qk, int d_v,
                            float scale, int causal, int deterministic,
                            void* workspace, size_t workspace_bytes, void* stream,
                            unsigned stages);

/*
 * Padded batches — the padding mask with per-batch query and key/value lengths
 * (seq_len_q, seq_len_kv) among the SDPA options of [SA8 1.2] — with the work of the
 * batch ordered by execution time, longest first, by a preprocessing kernel
 * [2CTA 3.2].
 *
 * Tensors keep their (B, NH, T, d) shapes and strides; T is the padded length.  Batch b
 * uses query rows 0 .. seq_len_q[b]-1 of q, o, do_, dq and key/value rows
 * 0 .. seq_len_kv[b]-1 of k, v, dk, dv; rows past them are padding.  Within a batch
 * the result is that of attn_fwd / attn_bwd on the unpadded rows, with the causal mask
 * top-left aligned (key j allowed for query i iff j <= i) also when the two lengths
 * differ.  Padding rows are never read and are written as: O = 0, LSE = -inf,
 * dQ = 0 (query padding); dK = dV = 0 (key padding).  A batch with seq_len_kv[b] = 0
 * has no keys: O = 0, LSE = -inf and zero gradients on all its rows.
 *
 *   seq_len_q, seq_len_kv : device pointers to B int32 each, 4-byte aligned (read);
 *                           values are clamped to [0, T] on the device (the host
 *                           cannot see them).  NULL: ATTN_ERR_NULL.
 *   workspace             : device memory of at least the matching *_workspace_bytes,
 *                           16-byte aligned, owned by the caller, clobbered; it holds
 *                           the sorted work lists (and, backward, what attn_bwd keeps
 *                           there).  Smaller or misaligned: ATTN_ERR_WORKSPACE.
 * Every other argument, layout rule and error is that of attn_fwd / attn_bwd.
 */
size_t attn_fwd_varlen_workspace_bytes(int B, int NH, int T, int d_qk, int d_v);

attn_status attn_fwd_varlen(const void* q, attn_strides sq,
                            const void* k, attn_strides sk,
                            const void* v, attn_strides sv,
                            void* o, attn_strides so,
                            float* lse,
                            const int32_t* seq_len_q, const int32_t* seq_len_kv,
                            int B, int NH, int T, int d_qk, int d_v,
                            float scale, int causal,
                            void* workspace, size_t workspace_bytes, void* stream);

size_t attn_bwd_varlen_workspace_bytes(int B, int NH, int T, int d_qk, int d_v, int deterministic);

attn_status attn_bwd_varlen(const void* q, attn_strides sq,
                            const void* k, attn_strides sk,
                            const void* v, attn_strides sv,
                            const void* o, attn_strides so,
                            const float* lse,
                            const void* do_, attn_strides sdo,
                            void* dq, attn_strides sdq,
                            void* dk, attn_strides sdk,
                            void* dv, attn_strides sdv,
                            const int32_t* seq_len_q, const int32_t* seq_len_kv,
                            int B, int NH, int T, int d_qk, int d_v,
                            float scale, int causal, int deterministic,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * 16-bit element types.  The pages run attention with 16-bit inputs and outputs and
 * fp32 accumulation, naming both fp16 and bf16 [SA8 1.3]; every entry point above takes
 * bf16.  The entry points below take either type, named by `dtype`, for all of q, k,
 * v, o, do_, dq, dk and dv of one call (LSE, D and the workspace stay fp32).  With fp16,
 * P and dS are rounded to fp16 (nearest even) before their products, as they are to bf16
 * in the bf16 path; the arithmetic is otherwise the same.
 */
typedef enum {
  ATTN_DTYPE_BF16 = 0,  /* bfloat16 (8-bit exponent, 8-bit significand) */
  ATTN_DTYPE_F16 = 1    /* IEEE binary16 (5-bit exponent, 11-bit significand) */
} attn_dtype;

/*
 * Sliding window (`window` argument of the two entry points below).  0: no window.
 * W >= 1: a banded causal mask, query i sees keys i-W+1 .. i only — the simplest of the
 * block-sparse mask patterns that the FA4 framework composes with causal masking
 * [2CTA 5.1, 5.2].  Tiles wholly outside the band are never loaded; only tiles that the
 * band's edges cross carry a mask.  W >= 1 needs causal = 1 and no padded-batch lengths,
 * W < 0 is invalid: otherwise ATTN_ERR_ARG.  Every row keeps at least its own key, so
 * the LSE and the outputs stay finite; the backward must get the forward's window.
 *
 * ALiBi bias (`alibi` argument of the two entry points below; the use_alibi_mask option
 * of [SA8 1.2]).  0: none.  1: the scaled scores get the linear bias -m_h (i - j) for
 * query i, key j <= i of head h, with the slopes m_h = 2^(-8 (h + 1) / NH) (the page
 * names the option, not its slopes; this geometric sequence is the reading taken).  The
 * bias is a constant of the inputs: it changes P, not the gradient formulas.  alibi = 1
 * needs causal = 1, no padded-batch lengths and window = 0; other values are invalid:
 * otherwise ATTN_ERR_ARG.  The backward must get the forward's flag.
 */

/*
 * attn_fwd_typed — attn_fwd (seq_len_q == seq_len_kv == NULL; workspace unused and may
 * be NULL) or attn_fwd_varlen (both lengths given; workspace as for attn_fwd_varlen) on
 * tensors of element type `dtype`, with an optional sliding window or ALiBi bias.  An unknown dtype
 * returns ATTN_ERR_ARG; every other argument, layout rule and error is that of
 * attn_fwd / attn_fwd_varlen.
 */
attn_status attn_fwd_typed(attn_dtype dtype,
                           const void* q, attn_strides sq,
                           const void* k, attn_strides sk,
                           const void* v, attn_strides sv,
                           void* o, attn_strides so,
                           float* lse,
                           const int32_t* seq_len_q, const int32_t* seq_len_kv,
                           int B, int NH, int T, int d_qk, int d_v,
                           float scale, int causal, int window, int alibi,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_typed — attn_bwd_staged (seq_len_q == seq_len_kv == NULL) or the padded-batch
 * backward (both lengths given) on tensors of element type `dtype`, with the forward's
 * sliding window (0 = none) and ALiBi flag, restricted to the
 * stages in `stages` (ATTN_BWD_ALL for the whole backward).  The workspace is sized by
 * attn_bwd_workspace_bytes / attn_bwd_varlen_workspace_bytes, which do not depend on the
 * element type.  An unknown dtype returns ATTN_ERR_ARG; every other argument, layout rule
 * and error is that of attn_bwd_staged / attn_bwd_varlen.
 */
attn_status attn_bwd_typed(attn_dtype dtype,
                           const void* q, attn_strides sq,
                           const void* k, attn_strides sk,
                           const void* v, attn_strides sv,
                           const void* o, attn_strides so,
                           const float* lse,
                           const void* do_, attn_strides sdo,
                           void* dq, attn_strides sdq,
                           void* dk, attn_strides sdk,
                           void* dv, attn_strides sdv,
                           const int32_t* seq_len_q, const int32_t* seq_len_kv,
                           int B, int NH, int T, int d_qk, int d_v,
                           float scale, int causal, int window, int alibi, int deterministic,
                           void* workspace, size_t workspace_bytes, void* stream,
                           unsigned stages);

/*
 * attn_fwd_decode — the inference-shaped forward of a decode step [SA8 1.2, 1.3]: Tq
 * query rows per sequence (the newest tokens) attend to all Tk key/value rows of that
 * sequence's cache, no causal mask among them (every query sees every cached key), in
 * the pages' inference mode when lse is NULL.  Tq and Tk are separate sizes:
 *   q     : (B, NH, Tq, d_qk), strides sq             (read)
 *   k, v  : (B, NH, Tk, d_qk / d_v), strides sk, sv   (read)
 *   o     : (B, NH, Tq, d_v), strides so              (written)
 *   lse   : (B, NH, Tq) fp32 contiguous, or NULL      (written)
 *   seq_len_kv : NULL (every cache holds Tk rows) or B int32 on the device, clamped to
 *                [0, Tk]: sequence b attends to its first seq_len_kv[b] key rows; with
 *                0 rows its O is 0 and its LSE -inf.
 * A workgroup owns 128 query rows of one (b, h) and streams the whole cache once;
 * wavefronts whose rows are all past Tq skip the arithmetic, so a one-row decode step
 * costs the cache read.  With fewer than 512 such workgroups the cache is split into
 * chunks of keys (at least 1024 keys each, at most 64 chunks) processed by workgroups
 * of their own; each writes its normalised fp32 partial O and LSE, and a merge kernel
 * combines them in one fixed order: O = sum_c e^(LSE_c - LSE) O_c, LSE = ln sum_c e^(LSE_c).
 *   workspace : device memory of at least attn_fwd_decode_workspace_bytes(...) bytes
 *               (0 when no split is needed; then it may be NULL), 16-byte aligned,
 *               owned by the caller, clobbered.  Too small: ATTN_ERR_WORKSPACE.
 * dtype, layout rules and errors as for attn_fwd_typed.
 */
size_t attn_fwd_decode_workspace_bytes(int B, int NH, int Tq, int Tk, int d_qk, int d_v);

attn_status attn_fwd_decode(attn_dtype dtype,
                            const void* q, attn_strides sq,
                            const void* k, attn_strides sk,
                            const void* v, attn_strides sv,
                            void* o, attn_strides so,
                            float* lse,
                            const int32_t* seq_len_kv,
                            int B, int NH, int Tq, int Tk, int d_qk, int d_v,
                            float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-sparse attention — the block-sparse mask pattern of the FA4 framework, a mask
 * module composed with the causal mask and with unchanged compute and scheduling
 * [2CTA 5.1, 5.2].  The pages give no format; this is the reading taken:
 *   block_map : device pointer to uint8 entries, one per (query block, key block) pair of
 *               128 x 128 elements, nb = ceil(T / 128) blocks along each side.  The map of
 *               head (b, h) starts at block_map + b * map_stride_b + h * map_stride_h
 *               (strides in bytes, >= 0; 0 shares one map across batches / heads) and is
 *               row-major (nb, nb): entry [qb * nb + kb].  Non-zero = live.  Read only.
 *   Element (i, j) is attended iff map[i / 128][j / 128] != 0 and, when causal = 1,
 *   j <= i.  Key blocks that are not live are never loaded; a live block that the
 *   causal mask or the end of the sequence cuts is a "partial" block and carries the
 *   element mask, every other live block is "full" and runs mask-free.  A query row left
 *   with no key gets O = 0 and LSE = -inf, and zero gradients; a key no query attends
 *   gets dK = dV = 0.
 *   workspace : device memory of at least the matching *_workspace_bytes, 16-byte
 *               aligned, owned by the caller, clobbered.  It holds the lists of live
 *               blocks that a preprocessing kernel builds from the map for every work
 *               item, and the work list ordered by cost, longest first [2CTA 3.2]
 *               (forward: about 4 * B * NH * nb * (nb + 3) bytes; the backward twice that
 *               plus what attn_bwd keeps there).  Too small: ATTN_ERR_WORKSPACE.
 * Element type bf16 (as attn_fwd / attn_bwd); every other argument, layout rule and error
 * is that of attn_fwd / attn_bwd_staged (map NULL: ATTN_ERR_NULL; a negative map stride:
 * ATTN_ERR_STRIDE; an output overlapping the map: ATTN_ERR_ALIAS).  The backward must
 * get the forward's map and causal flag.
 */
size_t attn_fwd_blocksparse_workspace_bytes(int B, int NH, int T, int d_qk, int d_v);

attn_status attn_fwd_blocksparse(const void* q, attn_strides sq,
                                 const void* k, attn_strides sk,
                                 const void* v, attn_strides sv,
                                 void* o, attn_strides so,
                                 float* lse,
                                 const uint8_t* block_map, int64_t map_stride_b, int64_t map_stride_h,
                                 int B, int NH, int T, int d_qk, int d_v,
                                 float scale, int causal,
                                 void* workspace, size_t workspace_bytes, void* stream);

size_t attn_bwd_blocksparse_workspace_bytes(int B, int NH, int T, int d_qk, int d_v, int deterministic);

attn_status attn_bwd_blocksparse(const void* q, attn_strides sq,
                                 const void* k, attn_strides sk,
                                 const void* v, attn_strides sv,
                                 const void* o, attn_strides so,
                                 const float* lse,
                                 const void* do_, attn_strides sdo,
                                 void* dq, attn_strides sdq,
                                 void* dk, attn_strides sdk,
                                 void* dv, attn_strides sdv,
                                 const uint8_t* block_map, int64_t map_stride_b, int64_t map_stride_h,
                                 int B, int NH, int T, int d_qk, int d_v,
                                 float scale, int causal, int deterministic,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 unsigned stages);

/*
 * Key bias — the attention bias of the SDPA options [SA8 1.2] (`bias`, `set_bias`), whose
 * shape the page does not give; read as a per-key additive bias broadcast over the
 * queries (which covers key-padding masks):
 *   S_ij = scale * <q_i, k_j> + bias[b, h, j],   dbias[b, h, j] = sum_i dS_ij
 * summed further over the batches / heads that share one bias row.
 *   bias  : fp32 device pointer, 4-byte aligned (read): bias + b * bias_stride_b +
 *           h * bias_stride_h + j for key j of head (b, h); strides in elements, >= 0, 0 to
 *           share one row across batches / heads; contiguous along the keys.  Values must be
 *           finite: mask a key with a large negative value (e.g. -1e9), not -inf.
 *   dbias : fp32 device pointer with the bias's strides (written; attn_bwd_keybias only),
 *           or NULL when no bias gradient is wanted.  Each element is the sum over its
 *           (b, h) pairs in one fixed order, so it is bit-stable; distinct elements must
 *           not share memory (ATTN_ERR_STRIDE).
 *   workspace : at least the matching *_workspace_bytes (the bias divided by the scale,
 *               B * NH * Tpad fp32; the backward adds the per-head sums of dS and what
 *               attn_bwd keeps there), 16-byte aligned, owned by the caller, clobbered.
 * Element type bf16; every other argument, layout rule and error is that of attn_fwd /
 * attn_bwd_staged (bias NULL: ATTN_ERR_NULL; an output overlapping the bias:
 * ATTN_ERR_ALIAS).  The backward must get the forward's bias and causal flag.
 */
size_t attn_fwd_keybias_workspace_bytes(int B, int NH, int T, int d_qk, int d_v);

attn_status attn_fwd_keybias(const void* q, attn_strides sq,
                             const void* k, attn_strides sk,
                             const void* v, attn_strides sv,
                             void* o, attn_strides so,
                             float* lse,
                             const float* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                             int B, int NH, int T, int d_qk, int d_v,
                             float scale, int causal,
                             void* workspace, size_t workspace_bytes, void* stream);

size_t attn_bwd_keybias_workspace_bytes(int B, int NH, int T, int d_qk, int d_v, int deterministic);

attn_status attn_bwd_keybias(const void* q, attn_strides sq,
                             const void* k, attn_strides sk,
                             const void* v, attn_strides sv,
                             const void* o, attn_strides so,
                             const float* lse,
                             const void* do_, attn_strides sdo,
                             void* dq, attn_strides sdq,
                             void* dk, attn_strides sdk,
                             void* dv, attn_strides sdv,
                             const float* bias, float* dbias, int64_t bias_stride_b, int64_t bias_stride_h,
                             int B, int NH, int T, int d_qk, int d_v,
                             float scale, int causal, int deterministic,
                             void* workspace, size_t workspace_bytes, void* stream,
                             unsigned stages);

/*
 * attn_fwd_fp8 — the forward on fp8 inputs, the FP8 lever of [FAT 5.3.4, 6] (less memory
 * traffic and twice the bf16 matrix rate); the pages give no recipe, so this is the
 * reading taken:
 *   q, k, v : e4m3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest
 *             finite 448, no infinity), (B, NH, T, d) through strides in elements (= bytes),
 *             16-byte aligned, strides multiples of 16 (read).  The real inputs are
 *             descale_q * q, descale_k * k, descale_v * v (per-tensor fp32 factors, finite,
 *             > 0; a caller typically picks descale = max|x| / 448).
 *   o       : bf16 (B, NH, T, d), strides so (written); lse as for attn_fwd (natural-log
 *             logsumexp of the scaled scores; NULL for inference).
 *   d_qk = d_v = 64 or 128 (otherwise ATTN_ERR_HEADDIM); causal 0 / 1.
 * S = scale descale_q descale_k Q K^T is formed exactly in fp32 by the fp8 matrix
 * instruction; P is rounded to e4m3 for O = P V (P <= 2^8 by the lazy-rescale rule, inside
 * e4m3's range), while the row sum adds the unrounded fp32 P; O = descale_v P V / l.  The
 * rounding of P (3 mantissa bits) is the path's one approximation beyond the fp32 sums.
 *   workspace : at least attn_fwd_fp8_workspace_bytes(...) bytes (a transposed copy of v,
 *               B * NH * d * ceil(T / 64) * 64 bytes, which the call writes first),
 *               16-byte aligned, owned by the caller, clobbered.
 * Forward only: the backward takes 16-bit tensors.  Other rules as for attn_fwd.
 */
size_t attn_fwd_fp8_workspace_bytes(int B, int NH, int T, int d_qk, int d_v);

attn_status attn_fwd_fp8(const void* q, attn_strides sq,
                         const void* k, attn_strides sk,
                         const void* v, attn_strides sv,
                         void* o, attn_strides so,
                         float* lse,
                         float descale_q, float descale_k, float descale_v,
                         int B, int NH, int T, int d_qk, int d_v,
                         float scale, int causal,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dropout on the attention weights — the `dropout` option of the SDPA interface
 * [SA8 1.2] (`set_dropout`), whose form the page does not give; read as inverted dropout
 * on P, with the keep decisions drawn from a counter-based generator:
 *   O = (P * Z) V / (1 - p),  LSE from the undropped P,
 *   dV = (P * Z)^T dO / (1 - p),  dP = (dO V^T) * Z / (1 - p),  dS = P * (dP - D),
 * D = rowsum(dO * O) as without dropout (O being the dropped output).
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with key = seed (low word
 * first).  Element (i, j) of head (b, h) takes 16-bit value j % 8 of the output at counter
 * (j / 8, i, b * NH + h, offset) — word (j % 8) / 2, low half for even j — and is kept iff
 * that value >= round(p * 65536) (p is quantised to 1/65536).
 *
 * attn_dropout_mask writes the keep bits once per step into a caller-owned buffer of
 * attn_dropout_mask_bytes(B, NH, T) bytes (two layouts of one bit per element, query-major
 * and key-major, each B * NH * Tp * Tp / 8 bytes with Tp = T rounded up to 128; 16-byte
 * aligned); causal = 1 leaves out blocks wholly above the diagonal.  attn_fwd_dropout and
 * attn_bwd_dropout read it (inputs; outputs must not overlap it) and must get the same p,
 * causal flag and sizes.  p in [0, 1) (otherwise ATTN_ERR_ARG); bf16; every other argument,
 * layout rule and error is that of attn_fwd / attn_bwd_staged.  The results are
 * bit-stable in the deterministic mode for one seed and offset.
 */
size_t attn_dropout_mask_bytes(int B, int NH, int T);

attn_status attn_dropout_mask(float p_drop, uint64_t seed, uint32_t offset,
                              int B, int NH, int T, int causal,
                              void* mask, size_t mask_bytes, void* stream);

attn_status attn_fwd_dropout(const void* q, attn_strides sq,
                             const void* k, attn_strides sk,
                             const void* v, attn_strides sv,
                             void* o, attn_strides so,
                             float* lse,
                             const void* mask, float p_drop,
                             int B, int NH, int T, int d_qk, int d_v,
                             float scale, int causal, void* stream);

attn_status attn_bwd_dropout(const void* q, attn_strides sq,
                             const void* k, attn_strides sk,
                             const void* v, attn_strides sv,
                             const void* o, attn_strides so,
                             const float* lse,
                             const void* do_, attn_strides sdo,
                             void* dq, attn_strides sdq,
                             void* dk, attn_strides sdk,
                             void* dv, attn_strides sdv,
                             const void* mask, float p_drop,
                             int B, int NH, int T, int d_qk, int d_v,
                             float scale, int causal, int deterministic,
                             void* workspace, size_t workspace_bytes, void* stream,
                             unsigned stages);

/*
 * attn_bwd_noalloc — attn_bwd without a caller-supplied workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, allocation-free serving or
 * training loops, harnesses that forbid hipMalloc.  The workspace (D, LSE log2(e) and, in
 * atomic mode, the fp32 dQ accumulator) lives in a static device array of the library,
 * attn_bwd_noalloc_max_workspace_bytes() = 64 MiB on each GPU, held from the library's
 * first use on that GPU until the process ends.  Every other argument, layout rule,
 * result and error is that of attn_bwd (the same kernels run).
 *   - Sizes whose attn_bwd_workspace_bytes(...) exceeds the maximum are rejected with
 *     ATTN_ERR_WORKSPACE before anything is launched (deterministic mode: 8 bytes per
 *     row of B * NH * Tpad, i.e. up to 8M padded rows; atomic mode adds 4 * d_qk bytes
 *     per row).
 *   - Allocates nothing: no hipMalloc, no hipFree, no allocating library call.  The
 *     kernels clear every part of the array they read before reading it.
 *   - All calls on one GPU share its array: calls that overlap in time on one GPU
 *     (different streams or threads without ordering between them) race and give
 *     undefined results.  Calls ordered on one stream are safe.
 */
size_t attn_bwd_noalloc_max_workspace_bytes(void);

attn_status attn_bwd_noalloc(const void* q, attn_strides sq,
                             const void* k, attn_strides sk,
                             const void* v, attn_strides sv,
                             const void* o, attn_strides so,
                             const float* lse,
                             const void* do_, attn_strides sdo,
                             void* dq, attn_strides sdq,
                             void* dk, attn_strides sdk,
                             void* dv, attn_strides sdv,
                             int B, int NH, int T, int d_qk, int d_v,
                             float scale, int causal, int deterministic, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN53_H */
