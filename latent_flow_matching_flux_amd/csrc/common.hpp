// Device-side helpers shared by the gfx950 kernels of libflux3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flux3 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16-byte raw chunk; a native vector type so arrays of it stay in registers
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// 32 fp8 codes: one lane's operand of the 32x32x64 fp8 MFMA
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kHeadDim = 128;
constexpr int kRopePairs = 64;        // 128 dims -> 64 rotated pairs
constexpr int kMaxSegs = 16;

// Per-call segment table passed by value to kernels that need the token ->
// segment map (modulation rows, gates).
struct SegTable {
  int32_t start[kMaxSegs];
  int32_t n;
};

__device__ __forceinline__ int seg_of(const SegTable& st, int m) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i)
    if (i < st.n && m >= st.start[i]) s = i;
  return s;
}

// One group of a launch's RowGroups, as a tile of workspace rows sees it:
// workspace row r holds token x0 + (r - ws0) when r - ws0 < n (live), and is
// padding otherwise; token() clamps padding rows to the group's last token
// (for loads whose results are discarded).
struct RowMap {
  int ws0, x0, n, w;
  __device__ __forceinline__ bool live(int r) const { return r - ws0 < n; }
  __device__ __forceinline__ int token(int r) const { return x0 + min(r - ws0, n - 1); }
};

// The group holding workspace row r (groups ascend in workspace rows).
template <class RG>
__device__ __forceinline__ RowMap row_map(const RG& rg, int r) {
  int g = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i)
    if (i < rg.n && r >= rg.ws_start[i]) g = i;
  return RowMap{rg.ws_start[g], rg.x_start[g], rg.count[g], rg.wsel[g]};
}

// 32x32x16 bf16 MFMA, fp32 accumulate.  Output layout (per lane l, reg r):
// column l % 32, row 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32x32x64 fp8 (e4m3 x e4m3) MFMA, fp32 accumulate, no block scaling (the
// scale operands 0 select the unscaled instruction).  Lane l supplies row
// l % 32 of A (column of B) and 32 of the 64 k-values; A and B use the same
// lane -> k assignment, so any fixed split of a row's 64 values over the two
// lane halves gives the same sum.  Output layout as mfma32.  The unit's
// internal sum is narrower than fp32: products far below the largest one of
// a group lose their low bits (measured: terms 2^-16 of the largest vanish,
// 2^-12 survive), an error of at most a few 2^-12 of the largest product.
__device__ __forceinline__ f32x16 mfma32_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// e4m3 codes of a * mult .. d * mult in bytes 0..3: nearest value, ties to
// the even code, clamped to +-448 first (the conversion itself turns
// magnitudes from 464 up into NaN); the sign is kept, also on zero.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float mult) {
  const float ya = fminf(fmaxf(a * mult, -448.f), 448.f);
  const float yb = fminf(fmaxf(b * mult, -448.f), 448.f);
  const float yc = fminf(fmaxf(c * mult, -448.f), 448.f);
  const float yd = fminf(fmaxf(d * mult, -448.f), 448.f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ya, yb, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(yc, yd, lo, true);
}

// Rowwise e4m3 quantisation of a row with largest magnitude amax: the
// multiplier 448 / amax and the dequantisation scale amax / 448, both
// correctly rounded fp32 divisions; an all-zero row gets 0 and 0.
__device__ __forceinline__ void e4m3_row_scale(float amax, float& mult, float& scale) {
  mult = amax > 0.f ? 448.f / amax : 0.f;
  scale = amax / 448.f;
}

__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }
__device__ __forceinline__ bf16 f2bf(float v) { return (bf16)v; }  // RNE

// Packed operand layout of the bf16 activations the GEMMs read (the
// modulated LayerNorm output and the attention / SwiGLU concatenation).  A
// row-major [R][K] matrix (R % 8 == 0, K % 64 == 0) is stored as 1-KiB
// blocks of 8 rows x 64 k-values, block (row / 8, k / 64) at block index
// (row / 8) * (K / 64) + k / 64.  Inside a block row r8 = row % 8 takes 128
// bytes, and its 16-byte chunk c (k-values 8c .. 8c + 7 of the block) sits
// in slot c ^ ((row / 2) % 8) -- the XOR swizzle the GEMM keeps in LDS -- so
// one 64-lane global->LDS load moves a whole block from contiguous memory.
__host__ __device__ __forceinline__ size_t packed_index(size_t row, int k, int K) {
  return ((((row >> 3) * (size_t)(K >> 6)) + (size_t)(k >> 6)) << 9) + ((row & 7) << 6) +
         ((size_t)(((k >> 3) & 7) ^ ((int)(row >> 1) & 7)) << 3) + (size_t)(k & 7);
}

// Packed layout of the fp8 operands (rowwise e4m3 weights and activations):
// the bytes of an [R][K] code matrix sit where the packed layout above puts
// a bf16 [R][K / 2] matrix, so the GEMMs' loads move them unchanged -- 1-KiB
// blocks of 8 rows x 128 k, row r8 = row % 8 taking 128 bytes, 16-byte chunk
// c (k-values 16c .. 16c + 15 of the block) in slot c ^ ((row / 2) % 8).
// R % 8 == 0, K % 128 == 0.
__host__ __device__ __forceinline__ size_t packed8_index(size_t row, int k, int K) {
  return ((((row >> 3) * (size_t)(K >> 7)) + (size_t)(k >> 7)) << 10) + ((row & 7) << 7) +
         ((size_t)(((k >> 4) & 7) ^ ((int)(row >> 1) & 7)) << 4) + (size_t)(k & 15);
}

// Even split of a run of work items over G persistent workgroups (the
// stream-K tail of attention).  Units of nk items each (an attention query
// block's key tiles) lie end to end, unit t owning items [t nk, (t + 1) nk); range v covers items
// [start(v), start(v + 1)) with start(v) = floor(v total / G).  A unit cut
// by range boundaries leaves one partial result per range that touches it:
// a range's first segment in slot 2v, its last (when in another unit) in
// slot 2v + 1, so 2G slots cover any split.
struct SplitK {
  int64_t total;   // units * nk
  int G, nk;
  __device__ __forceinline__ int64_t start(int v) const { return total * v / G; }
  // range holding item s
  __device__ __forceinline__ int range_of(int64_t s) const {
    return (int)(((s + 1) * G - 1) / total);
  }
  __device__ __forceinline__ int slot(int v, int t) const {
    return 2 * v + (t == (int)(start(v) / nk) ? 0 : 1);
  }
};

// Physical workgroup id -> range: the workgroups one XCD runs (every 8th id)
// take consecutive ranges, so they work on neighbouring units.
__device__ __forceinline__ int range_of_block(int b, int G) {
  return (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
}

// Cross-lane exchange inside a wave (ds_bpermute based).
__device__ __forceinline__ float xor_lane(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

}  // namespace flux3
