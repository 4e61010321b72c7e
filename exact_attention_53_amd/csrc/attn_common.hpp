// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4 only).
//
// Pages cited (by title and section):
//   [SA8]  "ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析"
//   [2CTA] "深度学习反向传播优化：2-CTA MMA模式与内存访问优化"
//   [FAT]  "FlashAttention Triton实现中的内存访问模式优化与寄存器分配策略"
//
// Element types.  Every kernel is a template over its 16-bit element type E: bf16
// (__bf16) or fp16 (_Float16), the two 16-bit input formats of [SA8 1.3].  Loads, LDS
// tiles and transposed reads move 16-bit words and do not depend on E; only the matrix
// instruction, the fp32 -> E roundings and the dot products used for row sums do.
//
// Matrix-core conventions (v_mfma_f32_32x32x16_bf16 / _f16, one 64-lane wavefront; lane l,
// half g = l / 32):
//   A operand (32 x 16): lane l holds A[l % 32][8g .. 8g+7]
//   B operand (16 x 32): lane l holds B[8g .. 8g+7][l % 32]
//   accumulator (32 x 32, 16 fp32 per lane): element r of lane l is
//       D[8 (r / 4) + 4 g + (r % 4)][l % 32]
// A product whose accumulator is transposed so that its rows are the contraction
// index of the next product (P feeding P V, dS feeding dS K, ...) can feed that next
// product straight from registers: the 8 accumulator values r = 8m .. 8m+7 of one
// lane form a valid A/B operand fragment if the *other* operand lists its
// contraction index in the same order, {16m + 4g + 0..3, 16m + 4g + 8..11}.  The
// transposed LDS reads below produce exactly that order.
//
// LDS tiles.  A tile of R rows x C columns of 16-bit elements (C a multiple of 64) is stored as
// C/64 panels, each R rows of 128 bytes.  Within a row the eight 16-byte chunks are
// permuted by XOR with swz(row).  With 64 LDS banks of 4 bytes this makes both access
// patterns conflict-free:
//   * row reads  (ds_read_b128): 16 lanes read the same chunk of 16 consecutive rows;
//   * column reads (ds_read_b64_tr_b16): 32 lanes read 4 consecutive rows x 64 bytes.
// This is the permuted shared-memory layout that [FAT 3.3] recommends over copying a
// transposed K in HBM, re-derived for the gfx950 bank geometry.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace attn53 {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <class E>
using vec8 = E __attribute__((ext_vector_type(8)));
template <class E>
using vec4 = E __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define ATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------------
// matrix core
// ---------------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// acc + the sum of the eight values of x, by four v_dot2_f32_bf16 / _f16 with (1, 1).
__device__ __forceinline__ float sum_pairs(const bf16x8& x, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), one, acc, false);
}
__device__ __forceinline__ float sum_pairs(const f16x8& x, float acc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 one = {(f16)1.f, (f16)1.f};
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(x, x, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(x, x, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(x, x, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2(__builtin_shufflevector(x, x, 6, 7), one, acc, false);
}

// 8 consecutive accumulator values (r = 8m .. 8m+7) rounded to E (nearest even).
template <class E>
__device__ __forceinline__ vec8<E> pack8(const f32x16& acc, int m) {
  vec8<E> r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (E)acc[8 * m + e];
  return r;
}

// ---------------------------------------------------------------------------------
// special functions and cross-lane reductions
// ---------------------------------------------------------------------------------
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Calls f(std::integral_constant<int, I>{}) for I = B .. E-1, in order.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Ends a scheduling region: the compiler moves no instruction across it.
#define ATTN_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Value held by lane l ^ 32 combined with the own value (one v_permlane32_swap).
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------------
// instruction-scheduling groups (__builtin_amdgcn_sched_group_barrier masks)
// ---------------------------------------------------------------------------------
constexpr int kSchedMfma = 0x008;
constexpr int kSchedValu = 0x002 | 0x400;  // VALU including transcendental
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;
#define ATTN_SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// ---------------------------------------------------------------------------------
// swizzled LDS tiles (byte offsets relative to the tile base)
// ---------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t swz(uint32_t row) {
  return (((row >> 1) & 1u) << 2) | ((row >> 2) & 3u);
}

template <int ROWS>
__device__ __forceinline__ uint32_t tile_off(uint32_t row, uint32_t col) {
  const uint32_t panel = col >> 6, chunk = (col >> 3) & 7u, e = col & 7u;
  return panel * (ROWS * 128u) + row * 128u + ((chunk ^ swz(row)) << 4) + (e << 1);
}

// Per-lane address bases.  For the access patterns below the swizzled offset splits
// into a per-lane base, an XOR with a small compile-time constant and an immediate
// offset, because the row index only enters swz() through bits that the loop steps
// (multiples of 16 rows) never touch, and the stepped column bits are disjoint from
// the rest of the base.  Keeping the bases in a few registers (instead of one
// address per tile and step) is what keeps the kernels free of spills.
struct LdsLane {
  uint32_t row;   // row reads:    lq * 128 + ((g ^ swz(lq)) << 4)
  uint32_t col0;  // column reads: rows 4g + p/4     (p = lane % 16)
  uint32_t col1;  //               rows 4g + p/4 + 8
};
__device__ __forceinline__ LdsLane lds_lane(uint32_t lane) {
  const uint32_t lq = lane & 31u, g = lane >> 5, p = lane & 15u;
  const uint32_t cl = (((lane >> 4) & 1u) << 1) | ((p & 3u) >> 1);  // chunk bits 0-1 of the column
  const uint32_t r0 = 4u * g + (p >> 2), r1 = r0 + 8u;
  LdsLane L;
  L.row = lq * 128u + ((g ^ swz(lq)) << 4);
  L.col0 = r0 * 128u + ((cl ^ swz(r0)) << 4) + 8u * (p & 1u);
  L.col1 = r1 * 128u + ((cl ^ swz(r1)) << 4) + 8u * (p & 1u);
  return L;
}

// Row read: lane l gets columns 16 ks + 8 g .. +7 of row R0 + l % 32 (R0 % 16 == 0).
template <class E, int ROWS>
__device__ __forceinline__ vec8<E> lds_row8(const ATTN_LDS char* tile, const LdsLane& L, int R0, int ks) {
  const uint32_t off = (uint32_t)(ks >> 2) * (ROWS * 128u) + (uint32_t)R0 * 128u + (L.row ^ ((uint32_t)(ks & 3) << 5));
  return *reinterpret_cast<const ATTN_LDS vec8<E>*>(tile + off);
}

// Column read for an MFMA operand whose contraction index runs along the tile's rows.
// Returns, for lane l, the 8 values X[k][j] with j = j0 + (l % 32) and
// k = k0 + 4 g + {0..3, 8..11} (g = l / 32), k0 % 16 == 0, j0 % 32 == 0: two
// ds_read_b64_tr_b16.  Within each 16-lane group, lane p supplies the address of row
// (k0 + 4g + 8h + p / 4), columns j0 + 16 * ((l / 16) % 2) + 4 (p % 4) .. +3.
template <class E, int ROWS>
__device__ __forceinline__ vec8<E> lds_col8(const ATTN_LDS char* tile, const LdsLane& L, int k0, int j0) {
  const uint32_t x = (uint32_t)((j0 >> 5) & 1) << 6;
  const uint32_t base = (uint32_t)(j0 >> 6) * (ROWS * 128u) + (uint32_t)k0 * 128u;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(tile + base + (L.col0 ^ x)));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(tile + base + (L.col1 ^ x)));
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(vec8<E>, v);
}

// ---------------------------------------------------------------------------------
// direct global -> LDS tile loads (buffer_load_dwordx4 ... lds)
// ---------------------------------------------------------------------------------
// A tile of ROWS x COLS 16-bit elements (rows of a matrix with row stride `ld`
// elements) is written to LDS in the swizzled panel layout by NW wavefronts.  Wavefront w fills the
// 1 KB blocks w, w + NW, ...; a block is 8 rows x 128 bytes of one panel, and lane l
// of the wavefront lands at byte 16 l of it, so the lane fetches the global chunk that
// the swizzle puts there.  Each lane keeps one 32-bit byte offset per block; the tile
// enters through a buffer resource (uniform) whose size ends at the last valid row, so
// rows at or past the end of the matrix read as zeros.  Row strides are limited to
// 2^24 elements by the API, which keeps every offset within 32 bits.
constexpr int kBufferResourceWord3 = 0x00020000;  // raw buffer, gfx9-family format

template <int ROWS, int COLS, int NW>
struct DirectTile {
  static constexpr int LOADS = ROWS * COLS * 2 / 1024 / NW;
  static_assert(ROWS * COLS * 2 % (1024 * NW) == 0, "tile not divisible into wave blocks");
  uint32_t off[LOADS];

  __device__ __forceinline__ void init(int64_t ld, int w, int lane) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int blk = w + NW * i;
      const int r = 8 * (blk % (ROWS / 8)) + (lane >> 3);
      const int col = 64 * (blk / (ROWS / 8)) + 8 * ((lane & 7) ^ (int)swz((uint32_t)r));
      off[i] = (uint32_t)((r * ld + col) * 2);
    }
  }
  // tile = matrix + row0 * ld (uniform); valid = number of matrix rows from row0 on (>= 1).
  __device__ __forceinline__ void issue(const void* tile, int64_t ld, int valid, ATTN_LDS char* dst, int w) const {
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer-resource builtins exist only for the GPU target
    const int64_t rows = valid < ROWS ? valid : ROWS;
    const int64_t bytes = ((rows - 1) * ld + COLS) * 2;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)tile, (short)0, (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff), kBufferResourceWord3);
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (ATTN_LDS void*)(dst + (w + NW * i) * 1024), 16, off[i], 0, 0, 0);
#endif
  }
};

// 64 consecutive fp32 values src[0 .. 63] -> LDS dst[0 .. 63], one dword per lane of one
// wavefront, by a direct buffer->LDS load; values at or past `valid` read as zero.  (A
// buffer load rather than a global one: the compiler then keeps counting the LDS reads
// in flight instead of waiting for all of them.)
__device__ __forceinline__ void load_f32x64_lds(const float* src, int valid, ATTN_LDS float* dst, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, valid * 4, kBufferResourceWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (ATTN_LDS void*)dst, 4, (uint32_t)lane * 4u, 0, 0, 0);
#endif
}

// ---------------------------------------------------------------------------------
// global <-> LDS tile staging through registers
// ---------------------------------------------------------------------------------
// A tile of ROWS x COLS 16-bit elements starting at global row `row0` of a (T, COLS) matrix with
// row stride `ld` elements.  Rows >= T are filled with zeros.  NT threads cooperate;
// each holds CHUNKS 16-byte chunks.  Chunk x -> panel x / (ROWS * 8), row (x / 8) %
// ROWS, chunk-in-row x % 8: eight consecutive lanes read one 128-byte row segment.
template <int ROWS, int COLS, int NT>
struct TileStage {
  static constexpr int CHUNKS = ROWS * COLS / 8 / NT;
  static_assert(ROWS * COLS / 8 % NT == 0, "tile not divisible among threads");
  u32x4 v[CHUNKS];

  template <class E>
  __device__ __forceinline__ void load(const E* __restrict__ g, int64_t ld, int row0, int T, int tid) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int x = tid + NT * i;
      const int panel = x / (ROWS * 8), rem = x % (ROWS * 8);
      const int row = rem >> 3, col = panel * 64 + (rem & 7) * 8;
      const int gr = row0 + row;
      if (gr < T) {
        v[i] = *reinterpret_cast<const u32x4*>(g + (int64_t)gr * ld + col);
      } else {
        v[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(ATTN_LDS char* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int x = tid + NT * i;
      const int panel = x / (ROWS * 8), rem = x % (ROWS * 8);
      const int row = rem >> 3, col = panel * 64 + (rem & 7) * 8;
      *reinterpret_cast<ATTN_LDS u32x4*>(tile + tile_off<ROWS>(row, col)) = v[i];
    }
  }
};

// ---------------------------------------------------------------------------------
// work schedule: longest items first, heads grouped per XCD
// ---------------------------------------------------------------------------------
// Workgroup ids are handed to the 8 XCDs round robin (id % 8).  When the number of
// (batch, head) pairs is a multiple of 8, each XCD gets a contiguous group of heads,
// so the workgroups that share a head's K/V (forward) or Q/dO (backward) share one L2
// — the head/batch swizzle of [2CTA 3.2].  Within an XCD, ids run over `rank`
// (0 = longest item first) and then over the XCD's heads.
struct Item {
  int rank;  // 0 .. nrank-1, in dispatch order
  int bh;    // b * NH + h
};
__device__ __forceinline__ Item schedule(int bid, int nbh) {
  Item it;
  if ((nbh & 7) == 0) {
    const int xcd = bid & 7, local = bid >> 3, per = nbh >> 3;
    it.bh = xcd * per + local % per;
    it.rank = local / per;
  } else {
    it.bh = bid % nbh;
    it.rank = bid / nbh;
  }
  return it;
}

// Work item of a padded-batch launch: `list` holds (b, block) pairs sorted longest
// first (attn_plan.hip); the workgroup ids run over list entries and heads, with the
// heads grouped per XCD as in schedule() when NH is a multiple of 8.
struct ListItem {
  int b, h, blk;
};
__device__ __forceinline__ ListItem list_item(int bid, int NH, const int* list) {
  int h, r;
  if ((NH & 7) == 0) {
    const int xcd = bid & 7, local = bid >> 3, per = NH >> 3;
    h = xcd * per + local % per;
    r = local / per;
  } else {
    h = bid % NH;
    r = bid / NH;
  }
  return ListItem{list[2 * r], h, list[2 * r + 1]};
}

// ALiBi slope of head h of NH in log2 units: m_h log2(e), m_h = 2^(-8 (h + 1) / NH).
__device__ __forceinline__ float alibi_slope_log2(int h, int NH) {
  return __builtin_amdgcn_exp2f(-8.f * (float)(h + 1) / (float)NH) * kLog2e;
}

// Dropout keep bits of an 8-element operand fragment.  A fragment pack8(acc, h) of a
// 32 x 32 accumulator whose rows (the contraction index) are 8 a + 4 g + e holds, for
// e8 = 0..7, row 16 h + 8 (e8 / 4) + 4 g + e8 % 4; w holds one keep bit per row (bit k for
// row k) of that accumulator.  Returns the fragment's 8 bits, bit e8 for element e8.
__device__ __forceinline__ uint32_t keep_bits8(uint32_t w, int h, int g) {
  const uint32_t x = w >> (16 * h + 4 * g);
  return (x & 0xFu) | ((x >> 4) & 0xF0u);
}

// Elements of a 16-bit fragment whose keep bit is 0 are set to zero.
template <class E>
__device__ __forceinline__ vec8<E> drop8(const vec8<E>& x, uint32_t bits) {
  u32x4 w = __builtin_bit_cast(u32x4, x);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = (bits >> (2 * k)) & 1u, hi = (bits >> (2 * k + 1)) & 1u;
    w[k] &= (lo ? 0x0000FFFFu : 0u) | (hi ? 0xFFFF0000u : 0u);
  }
  return __builtin_bit_cast(vec8<E>, w);
}

// Valid rows of batch b, clamped to [0, T].
__device__ __forceinline__ int batch_len(const int* seq, int b, int T) { return min(max(seq[b], 0), T); }

}  // namespace attn53
