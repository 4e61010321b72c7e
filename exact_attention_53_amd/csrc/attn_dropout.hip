// Dropout keep masks: Philox4x32-10 bits in the two layouts the attention kernels read.
//
// Pages cited (by title and section):
//   [SA8]  "ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析" 1.2 (the dropout option of
//          the SDPA interface)
// Generator: Philox4x32-10 of Salmon, Moraes, Dror and Shaw ("Parallel random numbers: as
// easy as 1, 2, 3", SC'11): a 128-bit counter and a 64-bit key, ten rounds of two
// 32 x 32 -> 64-bit products; the key is bumped by two Weyl constants before every round
// but the first.  Element (i, j) of head bh takes 16-bit value j % 8 of the output at
// counter (j / 8, i, bh, offset) (word (j % 8) / 2, low half for even j) and is kept iff
// that value >= round(p * 65536).
//
// Layouts (Tp = T rounded up to 128, rows of Tp / 8 bytes, bit k of byte c = element 8c + k):
//   rowmask[bh][i][j / 8]  (query-major: the forward and dQ kernels, whose lanes own a query)
//   colmask[bh][j][i / 8]  (key-major: the key/value kernel, whose lanes own a key)
// One wavefront owns 64 query rows x 128 keys: each lane draws the 16 counters of its row
// (16 bytes, one row-major store); a ballot per key then gathers that key's 64 row bits
// into one key-major word.  Under the causal mask, blocks wholly above the diagonal are
// skipped (never read).
#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn53 {

struct PhiloxOut {
  uint32_t x[4];
};

__device__ __forceinline__ PhiloxOut philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                   uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // each 32 x 32 -> 64-bit product as one v_mad_u64_u32 rather than a low and a high multiply
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    // three-input XORs as single v_bitop3_b32 (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(hi1, c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(hi0, c3, k1, 0x96);
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return PhiloxOut{{c0, c1, c2, c3}};
}

__global__ __launch_bounds__(64) void dropout_mask_kernel(DropoutMaskParams p) {
  const int nrb = p.Tp / 64, nkb = p.Tp / 128;
  const int bid = blockIdx.x;
  const int bh = bid / (nrb * nkb), rb = (bid / nkb) % nrb, kb = bid % nkb;
  if (p.causal && kb * 128 > rb * 64 + 63) return;  // every key above every row
  const int lane = threadIdx.x;
  const uint32_t i = (uint32_t)(rb * 64 + lane);
  const int ld = p.Tp / 8;
  // 16 groups of 8 keys: one Philox call each, one byte of keep bits each
  uint32_t bytes[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int gi = 0; gi < 16; ++gi) {
    const uint32_t grp = (uint32_t)(kb * 16 + gi);
    const PhiloxOut o = philox4x32_10(grp, i, (uint32_t)bh, p.offset, p.key0, p.key1);
    uint32_t bits = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t u = (o.x[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      bits |= (u >= p.threshold ? 1u : 0u) << e;
    }
    bytes[gi >> 2] |= bits << (8 * (gi & 3));
  }
  unsigned char* rowm = p.mask + ((int64_t)bh * p.Tp + i) * ld + kb * 16;
  *reinterpret_cast<u32x4*>(rowm) = u32x4{bytes[0], bytes[1], bytes[2], bytes[3]};
  // key-major: key kk of the block gathers its 64 row bits with one ballot
  uint64_t mine0 = 0, mine1 = 0;
#pragma unroll
  for (int kk = 0; kk < 128; ++kk) {
    const uint64_t m = __ballot((bytes[kk >> 5] >> (kk & 31)) & 1u);
    if (kk < 64) {
      if (lane == kk) mine0 = m;
    } else {
      if (lane == kk - 64) mine1 = m;
    }
  }
  unsigned char* colm = p.mask + (int64_t)p.B * p.NH * p.Tp * ld;
  const int64_t key = (int64_t)kb * 128 + lane;
  *reinterpret_cast<u32x2*>(colm + ((int64_t)bh * p.Tp + key) * ld + rb * 8) =
      u32x2{(uint32_t)mine0, (uint32_t)(mine0 >> 32)};
  *reinterpret_cast<u32x2*>(colm + ((int64_t)bh * p.Tp + key + 64) * ld + rb * 8) =
      u32x2{(uint32_t)mine1, (uint32_t)(mine1 >> 32)};
}

hipError_t launch_dropout_mask(const DropoutMaskParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.B * p.NH * (p.Tp / 64) * (p.Tp / 128);
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)n), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn53
