// Work lists for padded batches and block-sparse maps.
//
// Pages cited (by title and section):
//   [2CTA] "深度学习反向传播优化：2-CTA MMA模式与内存访问优化" 3.2 (load balancing: a
//          preprocessing kernel orders the batch's work by execution time)
//   [SA8]  "ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析" 1.2 (padding mask with
//          per-batch query and key/value lengths)
//
// With per-batch lengths, or a block-sparse map, the work of an item is known only on the
// device.
// One workgroup costs every item (the number of 64-row tiles its loop visits), sorts the
// items by cost, longest first, with a counting sort in LDS, and writes the list that
// the attention kernels then walk in launch order.  Items of cost 0 (blocks wholly in
// the padding, or batches without keys) stay in the list, last: they write the zero
// rows of the padding.  The order of equal-cost items depends on the order of the LDS
// atomics; no result depends on it.
#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn53 {

constexpr int PLAN_NT = 1024;
constexpr int PLAN_BUCKETS = PLAN_NT;  // costs above PLAN_BUCKETS - 1 share the top bucket

__device__ __forceinline__ int item_cost(const PlanParams& p, int b, int blk) {
  if (p.counts != nullptr) {  // block-sparse: two tiles per live block
    const int nblk = (p.T + p.block - 1) / p.block;
    return 2 * p.counts[b * nblk + blk];
  }
  const int lq = batch_len(p.seq_q, b, p.T), lk = batch_len(p.seq_k, b, p.T);
  if (p.kind == PLAN_Q) {  // query block: key tiles of 64 up to its diagonal / Lk
    const int q0 = blk * p.block;
    if (q0 >= lq || lk == 0) return 0;
    const int kv_end = p.causal ? min(lk, q0 + p.block) : lk;
    return (kv_end + 63) / 64;
  }
  const int key0 = blk * p.block;  // key block: query steps of 64 from its diagonal on
  if (key0 >= lk || lq == 0) return 0;
  return max(0, (lq + 63) / 64 - (p.causal ? key0 / 64 : 0));
}

__global__ __launch_bounds__(PLAN_NT) void plan_kernel(PlanParams p) {
  __shared__ int cnt[PLAN_BUCKETS];
  __shared__ int scan[PLAN_BUCKETS];
  const int tid = threadIdx.x;
  const int nblk = (p.T + p.block - 1) / p.block;
  const int n = p.B * nblk;
  cnt[tid] = 0;
  __syncthreads();
  // bucket 0 holds the largest cost
  for (int r = tid; r < n; r += PLAN_NT) {
    const int c = min(item_cost(p, r / nblk, r % nblk), PLAN_BUCKETS - 1);
    atomicAdd(&cnt[PLAN_BUCKETS - 1 - c], 1);
  }
  __syncthreads();
  const int mine = cnt[tid];
  scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < PLAN_BUCKETS; off <<= 1) {  // inclusive prefix sum
    const int add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  cnt[tid] = scan[tid] - mine;  // first list position of bucket tid
  __syncthreads();
  for (int r = tid; r < n; r += PLAN_NT) {
    const int b = r / nblk, blk = r % nblk;
    const int c = min(item_cost(p, b, blk), PLAN_BUCKETS - 1);
    const int pos = atomicAdd(&cnt[PLAN_BUCKETS - 1 - c], 1);
    p.items[2 * pos] = b;
    p.items[2 * pos + 1] = blk;
  }
}

hipError_t launch_plan(const PlanParams& p, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn53
