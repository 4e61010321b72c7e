// Block-sparse maps: from the caller's (query block, key block) map to the lists of live
// blocks that the attention kernels walk.
//
// Pages cited (by title and section):
//   [2CTA] "深度学习反向传播优化：2-CTA MMA模式与内存访问优化" 5.1, 5.2 (block-sparse attention
//          as a mask module composed with unchanged compute and scheduling), 3.2 (work
//          ordered by execution time, longest first)
//
// The map holds one byte per (query block, key block) pair of kBsBlock x kBsBlock
// elements (non-zero = live).  Element (i, j) is attended iff its block is live and, under
// the causal mask, j <= i.  For each work item one wavefront scans the item's row (or
// column, or group of rows) of the map 64 blocks at a time, and writes the live blocks in
// the order the kernel visits them: a ballot gives the live lanes, a popcount of the
// lanes before each one its position.  Blocks that the causal mask empties (key blocks
// above a query block's diagonal block) are left out here, so the kernels never load
// them.
#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn53 {

__global__ __launch_bounds__(64) void bs_index_kernel(BsIndexParams p) {
  const int item = blockIdx.x;  // over nbh * nblk
  const int bh = item / p.nblk, blk = item % p.nblk;
  const int b = bh / p.NH, h = bh % p.NH;
  const unsigned char* m = p.map + b * p.msb + h * p.msh;
  const int lane = threadIdx.x, nb = p.nb;
  const uint64_t below = (1ull << lane) - 1ull;  // lanes before this one
  int* out = p.idx + (int64_t)item * nb;
  int count = 0;
  if (p.kind == 1) {
    // key block `blk`: live query blocks, ascending (causal: from the diagonal block on)
    for (int c = p.causal ? blk : 0; c < nb; c += 64) {
      const int qb = c + lane;
      const bool live = qb < nb && m[(int64_t)qb * nb + blk] != 0;
      const uint64_t mask = __ballot(live);
      if (live) out[count + __popcll(mask & below)] = qb;
      count += __popcll(mask);
    }
  } else {
    // one query-block row (kind 0) or a group of p.group rows (kind 2): live key blocks,
    // descending (causal: from the group's last diagonal block down)
    const int r0 = blk * p.group;
    const int r1 = min(nb, r0 + p.group);
    const int top = p.causal ? r1 - 1 : nb - 1;
    for (int c = top; c >= 0; c -= 64) {
      const int kb = c - lane;  // lane 0 holds the highest block of the chunk
      int bits = 0;
      if (kb >= 0)
        for (int r = r0; r < r1; ++r)
          if ((!p.causal || kb <= r) && m[(int64_t)r * nb + kb] != 0) bits |= 1 << (r - r0);
      const bool live = bits != 0;
      const uint64_t mask = __ballot(live);
      if (live) out[count + __popcll(mask & below)] = p.kind == 2 ? (kb | (bits << 16)) : kb;
      count += __popcll(mask);
    }
  }
  if (lane == 0) p.cnt[item] = count;
}

hipError_t launch_bs_index(const BsIndexParams& p, hipStream_t s) {
  hipLaunchKernelGGL(bs_index_kernel, dim3(p.nbh * p.nblk), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn53
