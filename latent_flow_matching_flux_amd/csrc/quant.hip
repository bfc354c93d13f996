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
// One workgroup of 512 threads per block of 8 rows.  The 8 rows' 16-byte
// chunks are read in memory order (thread t takes chunks t, t + 512, ...),
// kept in registers while the row maxima are reduced (lanes of one row
// differ in their low 3 bits; then across the 8 waves through LDS), then
// converted and stored, 8 codes per chunk.  HBM-bound: 2 bytes read and 1
// written per value.
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

constexpr int QT = 512;                     // threads per workgroup
constexpr int QCPT = kQuantMaxK / QT;       // 16-byte chunks per thread at most
static_assert(QT % 64 == 0 && kQuantMaxK % QT == 0, "chunk split");

// Memory chunk c (c < K) of row block rb of a packed bf16 [R][K] matrix:
// bf16 block c / 64, row 8 rb + (c / 8) % 8, slot c % 8, which holds the
// k-chunk slot ^ ((row / 2) % 8).
struct PackedSource {
  const bf16* p;
  int K;
  __device__ __forceinline__ const bf16* chunk(int64_t rb, int c, int& k) const {
    const int b = c >> 6, r8 = (c >> 3) & 7, slot = c & 7;
    const int64_t row = 8 * rb + r8;
    k = 64 * b + 8 * (slot ^ ((int)(row >> 1) & 7));
    return p + (rb * (K >> 6) + b) * 512 + r8 * 64 + slot * 8;
  }
};

// The same chunk numbering over a Linear-layout matrix [R][Ka + Kb] given
// as two column pieces: 8 threads take 128 contiguous bytes of one row.
struct LinearSource {
  const bf16* a;
  const bf16* b;
  int Ka, Kb;
  __device__ __forceinline__ const bf16* chunk(int64_t rb, int c, int& k) const {
    const int blk = c >> 6, r8 = (c >> 3) & 7, slot = c & 7;
    const int64_t row = 8 * rb + r8;
    k = 64 * blk + 8 * slot;
    return k < Ka ? a + row * Ka + k : b + row * Kb + (k - Ka);
  }
};

template <class SRC>
__global__ __launch_bounds__(QT) void k_quant_rows(SRC src, uint8_t* __restrict__ out_a, int Ka,
                                                   uint8_t* __restrict__ out_b, int Kb,
                                                   float* __restrict__ scale) {
  __shared__ float red[QT / 64][8];
  const int64_t rb = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r8 = (t >> 3) & 7;
  const int64_t row = 8 * rb + r8;
  const int K = Ka + Kb;
  u32x4 v[QCPT];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < QCPT; ++i) {
    const int c = t + QT * i;
    if (c < K) {
      int k;
      v[i] = *reinterpret_cast<const u32x4*>(src.chunk(rb, c, k));
      const bf16x8 h = *reinterpret_cast<const bf16x8*>(&v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(bf2f(h[e])));
    }
  }
  amax = fmaxf(amax, xor_lane(amax, 1));
  amax = fmaxf(amax, xor_lane(amax, 2));
  amax = fmaxf(amax, xor_lane(amax, 4));
  if ((lane & 7) == 0) red[wave][r8] = amax;
  __syncthreads();
  amax = 0.f;
#pragma unroll
  for (int w = 0; w < QT / 64; ++w) amax = fmaxf(amax, red[w][r8]);
  float mult, rscale;
  e4m3_row_scale(amax, mult, rscale);
  if (t < 64 && (t & 7) == 0) scale[row] = rscale;
#pragma unroll
  for (int i = 0; i < QCPT; ++i) {
    const int c = t + QT * i;
    if (c < K) {
      int k;
      (void)src.chunk(rb, c, k);
      const bf16x8 h = *reinterpret_cast<const bf16x8*>(&v[i]);
      u32x2 codes;
      codes[0] = e4m3x4(bf2f(h[0]), bf2f(h[1]), bf2f(h[2]), bf2f(h[3]), mult);
      codes[1] = e4m3x4(bf2f(h[4]), bf2f(h[5]), bf2f(h[6]), bf2f(h[7]), mult);
      uint8_t* dst = k < Ka ? out_a + packed8_index(row, k, Ka)
                            : out_b + packed8_index(row, k - Ka, Kb);
      *reinterpret_cast<u32x2*>(dst) = codes;
    }
  }
}

}  // namespace

hipError_t launch_quant_packed_rows(const void* in, void* out, float* scale, int M, int K,
                                    hipStream_t s) {
  const unsigned blocks = (unsigned)((M + 7) / 8);
  if (blocks == 0) return hipSuccess;
  PackedSource src{static_cast<const bf16*>(in), K};
  hipLaunchKernelGGL(k_quant_rows<PackedSource>, dim3(blocks), dim3(QT), 0, s, src,
                     static_cast<uint8_t*>(out), K, static_cast<uint8_t*>(nullptr), 0, scale);
  return hipGetLastError();
}

hipError_t launch_quant_weight_rows(const void* a, int Ka, const void* b, int Kb, void* out_a,
                                    void* out_b, float* scale, int R, hipStream_t s) {
  const unsigned blocks = (unsigned)(R / 8);
  if (blocks == 0) return hipSuccess;
  LinearSource src{static_cast<const bf16*>(a), static_cast<const bf16*>(b), Ka, Kb};
  hipLaunchKernelGGL(k_quant_rows<LinearSource>, dim3(blocks), dim3(QT), 0, s, src,
                     static_cast<uint8_t*>(out_a), Ka, static_cast<uint8_t*>(out_b), Kb, scale);
  return hipGetLastError();
}

}  // namespace flux3
