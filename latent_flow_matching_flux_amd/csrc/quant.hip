// Rowwise e4m3 quantisation for the rowwise-FP8 blocks (the rowwise-FP8
// single file of the Diffusers release post, section "Smaller GPUs, single
// files, and custom LoRA training"): each row of a matrix gets the scale
// a / 448 (a its largest magnitude) and the e4m3 codes of its values times
// 448 / a, nearest with ties to the even code, clamped to +-448.
//
// Two sources: the packed bf16 concatenation [o | act] that the attention
// and projection kernels write (quantised once per block, before K4), and
// Linear-layout bf16 weights (once per weight set; the output projection's
// two matrices wo and w_down share one scale per row, as one linear over
// [o | act]).  Output in the packed fp8 layout the GEMMs load.
//
// One wave per row, 4 rows per workgroup.  Lane l takes the row's 16-byte
// chunks l, l + 64, ... (8 values each): one load instruction of a wave
// covers 512 consecutive values of the row, the 128-byte pieces of 8 packed
// blocks (or 1 KiB of a Linear row).  The chunks stay in registers while
// the wave reduces the row maximum, then each becomes 8 codes; a store
// instruction of the wave fills the row's 128 bytes in 4 fp8 blocks.  No
// LDS and no barrier, and at most 32 chunks per lane, so several
// workgroups share a CU and one's loads overlap another's conversions.
// HBM-bound: 2 bytes read and 1 written per value.
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

constexpr int QROWS = 4;                    // rows (waves) per workgroup
constexpr int QMAXC = kQuantMaxK / 512;     // chunks per lane at most
static_assert(kQuantMaxK % 512 == 0, "chunk split");

// Chunk j (values 8j .. 8j + 7) of row `row` of a packed bf16 [R][K]
// matrix: bf16 block j / 8 of the row's 8-row block, logical chunk j % 8 in
// slot (j % 8) ^ ((row / 2) % 8).
struct PackedSource {
  const bf16* p;
  int K;
  __device__ __forceinline__ const bf16* chunk(int64_t row, int j) const {
    return p + ((row >> 3) * (K >> 6) + (j >> 3)) * 512 + (row & 7) * 64 +
           ((j & 7) ^ ((int)(row >> 1) & 7)) * 8;
  }
};

// The same over a Linear-layout matrix [R][Ka + Kb] given as two column
// pieces.
struct LinearSource {
  const bf16* a;
  const bf16* b;
  int Ka, Kb;
  __device__ __forceinline__ const bf16* chunk(int64_t row, int j) const {
    const int k = 8 * j;
    return k < Ka ? a + row * Ka + k : b + row * Kb + (k - Ka);
  }
};

// C: chunks per lane the registers hold (>= K / 512).
template <class SRC, int C>
__global__ __launch_bounds__(64 * QROWS) void k_quant_rows(SRC src, int rows,
                                                           uint8_t* __restrict__ out_a, int Ka,
                                                           uint8_t* __restrict__ out_b, int Kb,
                                                           float* __restrict__ scale) {
  const int64_t row = (int64_t)blockIdx.x * QROWS + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int nc = (Ka + Kb) >> 3;            // chunks in the row
  u32x4 v[C];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int j = lane + 64 * i;
    if (j < nc) {
      v[i] = *reinterpret_cast<const u32x4*>(src.chunk(row, j));
      const bf16x8 h = *reinterpret_cast<const bf16x8*>(&v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(bf2f(h[e])));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, xor_lane(amax, o));
  float mult, rscale;
  e4m3_row_scale(amax, mult, rscale);
  if (lane == 0) scale[row] = rscale;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int j = lane + 64 * i;
    if (j < nc) {
      const bf16x8 h = *reinterpret_cast<const bf16x8*>(&v[i]);
      u32x2 codes;
      codes[0] = e4m3x4(bf2f(h[0]), bf2f(h[1]), bf2f(h[2]), bf2f(h[3]), mult);
      codes[1] = e4m3x4(bf2f(h[4]), bf2f(h[5]), bf2f(h[6]), bf2f(h[7]), mult);
      const int k = 8 * j;
      uint8_t* dst = k < Ka ? out_a + packed8_index(row, k, Ka)
                            : out_b + packed8_index(row, k - Ka, Kb);
      *reinterpret_cast<u32x2*>(dst) = codes;
    }
  }
}

template <class SRC>
hipError_t launch_rows(const SRC& src, int rows, uint8_t* out_a, int Ka, uint8_t* out_b, int Kb,
                       float* scale, hipStream_t s) {
  const unsigned blocks = (unsigned)((rows + QROWS - 1) / QROWS);
  if (blocks == 0) return hipSuccess;
  const int c = (Ka + Kb + 511) / 512;      // chunks per lane
  const dim3 grid(blocks), block(64 * QROWS);
  if (c <= 4)
    hipLaunchKernelGGL((k_quant_rows<SRC, 4>), grid, block, 0, s, src, rows, out_a, Ka, out_b,
                       Kb, scale);
  else if (c <= 8)
    hipLaunchKernelGGL((k_quant_rows<SRC, 8>), grid, block, 0, s, src, rows, out_a, Ka, out_b,
                       Kb, scale);
  else if (c <= 16)
    hipLaunchKernelGGL((k_quant_rows<SRC, 16>), grid, block, 0, s, src, rows, out_a, Ka, out_b,
                       Kb, scale);
  else if (c <= 24)
    hipLaunchKernelGGL((k_quant_rows<SRC, 24>), grid, block, 0, s, src, rows, out_a, Ka, out_b,
                       Kb, scale);
  else
    hipLaunchKernelGGL((k_quant_rows<SRC, QMAXC>), grid, block, 0, s, src, rows, out_a, Ka,
                       out_b, Kb, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_packed_rows(const void* in, void* out, float* scale, int M, int K,
                                    hipStream_t s) {
  // whole 8-row blocks: the rows up to the next multiple of 8 (all inside
  // the n_pad rows of the buffers) get codes too
  PackedSource src{static_cast<const bf16*>(in), K};
  return launch_rows(src, (M + 7) / 8 * 8, static_cast<uint8_t*>(out), K,
                     static_cast<uint8_t*>(nullptr), 0, scale, s);
}

hipError_t launch_quant_weight_rows(const void* a, int Ka, const void* b, int Kb, void* out_a,
                                    void* out_b, float* scale, int R, hipStream_t s) {
  LinearSource src{static_cast<const bf16*>(a), static_cast<const bf16*>(b), Ka, Kb};
  return launch_rows(src, R, static_cast<uint8_t*>(out_a), Ka, static_cast<uint8_t*>(out_b), Kb,
                     scale, s);
}

}  // namespace flux3
