// Exact attention forward on fp8 (e4m3) inputs for gfx950.
//
// Pages cited (by title and section):
//   [FAT]  "FlashAttention Triton实现中的内存访问模式优化与寄存器分配策略" 5.3.4 and 6 (FP8 as the
//          lever that cuts memory traffic and compute), 2.2 (one program per query block,
//          running max / sum), 3.3 (a transposed copy made outside the kernel so that the
//          kernel's operand reads are row reads), 4.2 (deferred normalisation)
//   [SA8]  "ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析" 2.1, A.1 (S, P, O), 1.2 (stats)
//   [2CTA] "深度学习反向传播优化：2-CTA MMA模式与内存访问优化" 3.2, 6.2 (longest first, diagonal first)
//
// Q, K, V hold e4m3 codes; the real inputs are descale_q * Q, descale_k * K, descale_v * V.
// Both products run on the fp8 matrix instruction v_mfma_f32_32x32x64_f8f6f4 (twice the
// bf16 rate): lane l holds row l % 32 of its operand and 32 consecutive values of the
// contraction index, 32 (l / 32) .. +31; the accumulator layout is that of the bf16
// instruction (element r of lane l: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32).
//   * S^T = K Q^T: K rows from LDS (two 16-byte reads per operand), Q rows in registers;
//     descale_q descale_k scale log2(e) is folded into the exponent.
//   * p = 2^(S c - m) as in the 16-bit forward (lazy rescale, p <= 2^8 < 448, the largest
//     e4m3 value), rounded to e4m3 (v_cvt_pk_fp8_f32, nearest even) for O^T += V^T P^T;
//     the row sum l adds the unrounded fp32 p.  The S^T accumulator puts keys
//     8a + 4g + 0..3 (and 32 + ...) of a query in lane half g; four v_permlane32_swap of
//     packed fp8 words turn that into keys 32g .. 32g + 31 in order, the B-operand layout.
//   * V^T comes from a transposed copy of V in the workspace (one small kernel per call),
//     so the A operand of O^T += V^T P^T is a row read as well.
//   * O = descale_v O^T / l -> bf16; LSE = ln 2 (m + log2 l) of the scaled scores.
// LDS: 64-key K tiles (64 x d bytes) and V^T tiles (d x 64 bytes), double-buffered, filled
// by direct global->LDS loads into swizzled layouts: 128-byte rows use the 16-bit
// kernels' panel swizzle, 64-byte rows XOR the 16-byte chunk with bits 2-3 of the row,
// which makes both row-read patterns conflict-free.
#include <type_traits>

#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn53 {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int F8_BM = 128;
constexpr int F8_BN = 64;
constexpr int F8_NT = 256;
constexpr float kF8RescaleThreshold = 8.f;
constexpr float kF8SumLimit = 256.f;

__device__ __forceinline__ f32x16 mfma64(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);  // e4m3 x e4m3
}

// 16-byte chunk c of row r of a tile of 64-byte rows sits at r * 64 + 16 (c ^ ((r >> 2) & 3)).
__device__ __forceinline__ uint32_t swz64(uint32_t r) { return (r >> 2) & 3u; }

// Direct global -> LDS load of a tile of ROWS rows x 64 bytes (rows `ld` bytes apart) by NW
// wavefronts; rows at or past `valid` read as zero.  Wavefront w fills the 1 KB blocks
// w, w + NW, ... (16 rows each); lane l lands at byte 16 l of its block, so it fetches the
// global chunk that the swizzle puts there.
template <int ROWS, int NW>
struct DirectTile64B {
  static constexpr int LOADS = ROWS * 64 / 1024 / NW;
  static_assert(ROWS * 64 % (1024 * NW) == 0, "tile not divisible into wave blocks");
  uint32_t off[LOADS];
  __device__ __forceinline__ void init(int64_t ld, int w, int lane) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = 16 * (w + NW * i) + (lane >> 2);
      const int c = (lane & 3) ^ (int)swz64((uint32_t)r);
      off[i] = (uint32_t)(r * ld + 16 * c);
    }
  }
  __device__ __forceinline__ void issue(const void* tile, int64_t ld, int valid, ATTN_LDS char* dst, int w) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int64_t rows = valid < ROWS ? valid : ROWS;
    const int64_t bytes = (rows - 1) * ld + 64;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)tile, (short)0, (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff), kBufferResourceWord3);
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (ATTN_LDS void*)(dst + (w + NW * i) * 1024), 16, off[i], 0, 0, 0);
#endif
  }
};

// 32 consecutive bytes (two 16-byte reads) at two LDS byte addresses.
__device__ __forceinline__ i32x8 lds_32b(const ATTN_LDS char* base, uint32_t a0, uint32_t a1) {
  const u32x4 x = *reinterpret_cast<const ATTN_LDS u32x4*>(base + a0);
  const u32x4 y = *reinterpret_cast<const ATTN_LDS u32x4*>(base + a1);
  return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
}

// Four fp32 values -> one word of four e4m3 codes (byte e holds x[e]).
__device__ __forceinline__ int pack_fp8x4(float x0, float x1, float x2, float x3) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, v, true);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(F8_NT, 2) void fwd_fp8_kernel(Fp8FwdParams p) {
  constexpr int KS = D / 64;   // k-steps of 64 over the head dim
  constexpr int NDT = D / 32;  // 32-row tiles of O^T
  constexpr int KT_BYTES = F8_BN * D, VT_BYTES = D * F8_BN;
  __shared__ __attribute__((aligned(1024))) char kbuf0[KT_BYTES], kbuf1[KT_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[VT_BYTES], vbuf1[VT_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, lq = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T;
  const int nqb = (T + F8_BM - 1) / F8_BM;
  const Item item = schedule(blockIdx.x, p.B * p.NH);
  const int qb = CAUSAL ? nqb - 1 - item.rank : item.rank;
  const int bh = item.bh, b = bh / p.NH, h = bh % p.NH;

  const char* qg = (const char*)p.q + b * p.sq.b + h * p.sq.h;
  const char* kg = (const char*)p.k + b * p.sk.b + h * p.sk.h;
  const char* vtg = (const char*)p.vt + (int64_t)bh * D * p.vt_ld;
  bf16* og = (bf16*)p.o + b * p.so.b + h * p.so.h;
  const int64_t skt = p.sk.t;

  const int q0 = qb * F8_BM, qw = q0 + 32 * w, my_q = qw + lq;
  const int kv_end = CAUSAL ? min(T, q0 + F8_BM) : T;
  const int n_kv = (kv_end + F8_BN - 1) / F8_BN;

  // Q row of this lane: k-step ks holds bytes 64 ks + 32 g .. +31
  i32x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (my_q < T) {
      const char* src = qg + (int64_t)my_q * p.sq.t + 64 * ks + 32 * g;
      x = *reinterpret_cast<const u32x4*>(src);
      y = *reinterpret_cast<const u32x4*>(src + 16);
    }
    qf[ks] = i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
  }

  // LDS read addresses.  K rows (128-byte rows for d = 128: panel swizzle; 64-byte rows for
  // d = 64): chunks 2 g + hh of k-step ks; V^T rows: chunks 2 g + hh.
  uint32_t ka[2], va[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    if constexpr (D == 128)
      ka[hh] = lq * 128u + ((((uint32_t)(2 * g + hh)) ^ swz(lq)) << 4);
    else
      ka[hh] = lq * 64u + ((((uint32_t)(2 * g + hh)) ^ swz64(lq)) << 4);
    va[hh] = lq * 64u + ((((uint32_t)(2 * g + hh)) ^ swz64(lq)) << 4);
  }
  constexpr uint32_t KROW = D;  // bytes per K row in LDS

  // K tile loader: d = 128 reuses the 16-bit panel loader (64 columns of 16 bits = 128 bytes).
  using KLoad = typename std::conditional<D == 128, DirectTile<F8_BN, 64, F8_NT / 64>, DirectTile64B<F8_BN, F8_NT / 64>>::type;
  KLoad kload;
  DirectTile64B<D, F8_NT / 64> vload;
  kload.init(D == 128 ? skt / 2 : skt, w, lane);
  vload.init(p.vt_ld, w, lane);
  auto load_kv = [&](int key0, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    kload.issue(kg + key0 * skt, D == 128 ? skt / 2 : skt, T - key0, (ATTN_LDS char*)(BUF ? kbuf1 : kbuf0), w);
    vload.issue(vtg + key0, p.vt_ld, D, (ATTN_LDS char*)(BUF ? vbuf1 : vbuf0), w);
  };

  const float c = p.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = zero16();

  load_kv((n_kv - 1) * F8_BN, std::integral_constant<int, 0>{});

  auto step = [&](int it, auto bufc, auto maskc) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr bool MASKED = decltype(maskc)::value;
    const int j = n_kv - 1 - it;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 < n_kv) load_kv((j - 1) * F8_BN, std::integral_constant<int, 1 - BUF>{});
    const int key0 = j * F8_BN;
    if (MASKED && CAUSAL && key0 > qw + 31) return;  // tile wholly above this wavefront's rows
    const ATTN_LDS char* kt = (const ATTN_LDS char*)(BUF ? kbuf1 : kbuf0);
    const ATTN_LDS char* vt = (const ATTN_LDS char*)(BUF ? vbuf1 : vbuf0);
    f32x16 s0, s1;
    auto scores = [&]() __attribute__((always_inline)) {
      s0 = zero16();
      s1 = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t x = (uint32_t)ks << 6;  // chunk 4 ks (only with 128-byte rows)
        s0 = mfma64(lds_32b(kt, ka[0] ^ x, ka[1] ^ x), qf[ks], s0);
        s1 = mfma64(lds_32b(kt + 32 * KROW, ka[0] ^ x, ka[1] ^ x), qf[ks], s1);
      }
      if constexpr (MASKED) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk0 = key0 + 8 * (r >> 2) + 4 * g + (r & 3), kk1 = kk0 + 32;
          if (kk0 >= T || (CAUSAL && kk0 > my_q)) s0[r] = -INFINITY;
          if (kk1 >= T || (CAUSAL && kk1 > my_q)) s1[r] = -INFINITY;
        }
      }
    };
    auto tile_max = [&]() __attribute__((always_inline)) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s0[r], s1[r]));
      return max_halves(mx) * c;
    };
    auto raise_max = [&](float m_tile) __attribute__((always_inline)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    };
    auto probs = [&]() __attribute__((always_inline)) {
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = exp2_fast(__builtin_fmaf(s0[r], c, -m_run));
        s1[r] = exp2_fast(__builtin_fmaf(s1[r], c, -m_run));
        rs += s0[r] + s1[r];
      }
      return rs;
    };
    scores();
    float rs;
    if constexpr (MASKED) {
      const float m_tile = tile_max();
      if (__builtin_expect(__any(m_tile > m_run + kF8RescaleThreshold), 0)) {
        asm volatile("");
        raise_max(m_tile);
      }
      rs = probs();
    } else {
      rs = probs();
      if (__builtin_expect(__any(rs > kF8SumLimit), 0)) {
        asm volatile("");
        scores();
        raise_max(tile_max());
        rs = probs();
      }
    }
    l_run += rs;
    // P^T operand: e4m3 words of keys 8a + 4g + 0..3 (s0) and 32 + 8a + 4g + 0..3 (s1),
    // exchanged between the lane halves so that half g holds keys 32 g .. 32 g + 31.
    int y[4], x[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      y[a] = pack_fp8x4(s0[4 * a], s0[4 * a + 1], s0[4 * a + 2], s0[4 * a + 3]);
      x[a] = pack_fp8x4(s1[4 * a], s1[4 * a + 1], s1[4 * a + 2], s1[4 * a + 3]);
      const auto sw = __builtin_amdgcn_permlane32_swap((unsigned)y[a], (unsigned)x[a], false, false);
      y[a] = (int)sw[0];
      x[a] = (int)sw[1];
    }
    const i32x8 pf = {y[0], x[0], y[1], x[1], y[2], x[2], y[3], x[3]};
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = mfma64(lds_32b(vt + 32 * dt * 64, va[0], va[1]), pf, o[dt]);
  };

  constexpr auto B0 = std::integral_constant<int, 0>{};
  constexpr auto B1 = std::integral_constant<int, 1>{};
  const int first_ragged = T % F8_BN != 0 ? T / F8_BN : n_kv;
  const int first_masked = min(min(first_ragged, CAUSAL ? q0 / F8_BN : n_kv), n_kv);
  const int n_mask = n_kv - first_masked;
  int it = 0;
  if (qw >= T) {  // every row of this wavefront is past T: loads and barriers only
    for (; it < n_kv; ++it) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (it + 1 < n_kv) {
        if (it & 1)
          load_kv((n_kv - 2 - it) * F8_BN, B0);
        else
          load_kv((n_kv - 2 - it) * F8_BN, B1);
      }
    }
  } else {
    for (; it < n_mask; ++it) {
      if (it & 1)
        step(it, B1, std::true_type{});
      else
        step(it, B0, std::true_type{});
    }
    if ((it & 1) && it < n_kv) step(it++, B1, std::false_type{});
    for (; it + 1 < n_kv; it += 2) {
      step(it, B0, std::false_type{});
      step(it + 1, B1, std::false_type{});
    }
    if (it < n_kv) step(it++, B0, std::false_type{});
  }

  const float l_tot = sum_halves(l_run);
  if (my_q < T) {
    const float inv = p.descale_v / l_tot;
    bf16* orow = og + (int64_t)my_q * p.so.t;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        vec4<bf16> v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[dt][4 * a + e] * inv);
        *reinterpret_cast<vec4<bf16>*>(orow + 32 * dt + 8 * a + 4 * g) = v;
      }
    if (p.lse != nullptr && g == 0) p.lse[(int64_t)bh * T + my_q] = (m_run + log2_fast(l_tot)) * kLn2;
  }
}

// V (B, NH, T, d) e4m3 -> V^T (B * NH, d, ld) in the workspace, zero for t >= T.  One
// workgroup per (b, h, 64 keys), through LDS.
template <int D>
__global__ __launch_bounds__(256) void vt_kernel(Fp8FwdParams p) {
  __shared__ unsigned char tile[F8_BN][D + 16];
  const int nt = p.vt_ld / F8_BN;
  const int bh = blockIdx.x / nt, t0 = (blockIdx.x % nt) * F8_BN;
  const int b = bh / p.NH, h = bh % p.NH;
  const char* vg = (const char*)p.v + b * p.sv.b + h * p.sv.h;
  for (int x = threadIdx.x; x < F8_BN * D / 16; x += 256) {
    const int row = x / (D / 16), ch = x % (D / 16), t = t0 + row;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (t < p.T) val = *reinterpret_cast<const u32x4*>(vg + (int64_t)t * p.sv.t + 16 * ch);
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<unsigned*>(&tile[row][16 * ch + 4 * e]) = val[e];
  }
  __syncthreads();
  char* dst = (char*)p.vt + (int64_t)bh * D * p.vt_ld;
  for (int y = threadIdx.x; y < D * (F8_BN / 16); y += 256) {
    const int d = y / (F8_BN / 16), c16 = y % (F8_BN / 16);
    u32x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      val[e] = (unsigned)tile[16 * c16 + 4 * e][d] | ((unsigned)tile[16 * c16 + 4 * e + 1][d] << 8) |
               ((unsigned)tile[16 * c16 + 4 * e + 2][d] << 16) | ((unsigned)tile[16 * c16 + 4 * e + 3][d] << 24);
    *reinterpret_cast<u32x4*>(dst + (int64_t)d * p.vt_ld + t0 + 16 * c16) = val;
  }
}

template <int D>
static hipError_t fwd_fp8_t(const Fp8FwdParams& p, bool causal, hipStream_t s) {
  const int nt = p.vt_ld / F8_BN;
  hipLaunchKernelGGL((vt_kernel<D>), dim3(p.B * p.NH * nt), dim3(256), 0, s, p);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const dim3 grid((p.T + F8_BM - 1) / F8_BM * p.B * p.NH);
  if (causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, true>), grid, dim3(F8_NT), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, false>), grid, dim3(F8_NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, int d, bool causal, hipStream_t s) {
  if (d == 64) return fwd_fp8_t<64>(p, causal, s);
  if (d == 128) return fwd_fp8_t<128>(p, causal, s);
  return hipErrorInvalidValue;
}

}  // namespace attn53
