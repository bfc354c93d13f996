// K1: parameter-free LayerNorm + per-segment adaLN modulation.
//
// Every block starts with a LayerNorm that has no learned affine; the scale
// and shift come from the timestep embedding, per token type ("Speed,
// architecture, and how the tokens move", 15jq.com post; block listing of
// the Diffusers release post, everytik.com translation):
//   h = (1 + scale_s) * (x - mean) / sqrt(var + eps) + shift_s
// Statistics are fp32 over the row (biased variance, two passes over
// registers); h is written as bf16, the GEMM operand type, in the packed
// operand layout (1-KiB blocks of 8 rows x 64 k, chunks swizzled).
//
// One wave per row; each lane holds width/64 values.  HBM-bound: reads 4 B
// and writes 2 B per element (the modulation vectors stay in cache).  Rows
// are workspace rows: a grouped launch (RowGroups) maps each to its token
// and skips padding rows.
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

template <int D>
__global__ __launch_bounds__(256) void k_ln_modulate(
    const float* __restrict__ x, const float* __restrict__ mod, SegTable segs, RowGroups rg,
    bf16* __restrict__ h, int rows, float eps) {
  constexpr int V = D / (kWave * 4);  // float4 per lane
  const int lane = threadIdx.x & 63;
  const int wr = blockIdx.x * 4 + (threadIdx.x >> 6);   // workspace row
  if (wr >= rows) return;
  const RowMap g = row_map(rg, wr);
  if (!g.live(wr)) return;
  const int row = g.token(wr);
  const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * D);
  float4 v[V];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    v[i] = xr[lane + 64 * i];
    s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += xor_lane(s, o);
  const float mean = s * (1.0f / D);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean,
                d = v[i].w - mean;
    q += (a * a + b * b) + (c * c + d * d);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) q += xor_lane(q, o);
  const float rstd = 1.0f / sqrtf(q * (1.0f / D) + eps);

  const int sg = seg_of(segs, row);
  const float4* shift = reinterpret_cast<const float4*>(mod + (size_t)sg * 3 * D);
  const float4* scale = shift + D / 4;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int c = lane + 64 * i;
    const float4 sh = shift[c], sc = scale[c];
    bf16x4 o;
    o[0] = f2bf((1.0f + sc.x) * ((v[i].x - mean) * rstd) + sh.x);
    o[1] = f2bf((1.0f + sc.y) * ((v[i].y - mean) * rstd) + sh.y);
    o[2] = f2bf((1.0f + sc.z) * ((v[i].z - mean) * rstd) + sh.z);
    o[3] = f2bf((1.0f + sc.w) * ((v[i].w - mean) * rstd) + sh.w);
    *reinterpret_cast<bf16x4*>(h + packed_index(wr, 4 * c, D)) = o;
  }
}

// Generic width (any multiple of 256): loops instead of a register array.
__global__ __launch_bounds__(256) void k_ln_modulate_any(
    const float* __restrict__ x, const float* __restrict__ mod, SegTable segs, RowGroups rg,
    bf16* __restrict__ h, int rows, int D, float eps) {
  const int lane = threadIdx.x & 63;
  const int wr = blockIdx.x * 4 + (threadIdx.x >> 6);   // workspace row
  if (wr >= rows) return;
  const RowMap g = row_map(rg, wr);
  if (!g.live(wr)) return;
  const int row = g.token(wr);
  const float* xr = x + (size_t)row * D;
  float s = 0.f;
  for (int c = lane; c < D; c += 64) s += xr[c];
  for (int o = 32; o >= 1; o >>= 1) s += xor_lane(s, o);
  const float mean = s / (float)D;
  float q = 0.f;
  for (int c = lane; c < D; c += 64) {
    const float a = xr[c] - mean;
    q += a * a;
  }
  for (int o = 32; o >= 1; o >>= 1) q += xor_lane(q, o);
  const float rstd = 1.0f / sqrtf(q / (float)D + eps);
  const int sg = seg_of(segs, row);
  const float* shift = mod + (size_t)sg * 3 * D;
  const float* scale = shift + D;
  for (int c = lane; c < D; c += 64)
    h[packed_index(wr, c, D)] = f2bf((1.0f + scale[c]) * ((xr[c] - mean) * rstd) + shift[c]);
}

// Rowwise-fp8 output (blocks with e4m3 weights): the same h values in fp32,
// then the row's largest magnitude a, the codes of h * (448 / a) in the
// packed fp8 layout and the row scale a / 448.  One wave per row.  Any width
// that is a multiple of 256; at 3072 the row stays in registers, otherwise
// the values are recomputed from x for each pass.
template <int V>
__device__ __forceinline__ void ln_row_f8(const float* __restrict__ x, const float* __restrict__ mod,
                                          const SegTable& segs, uint8_t* __restrict__ h8,
                                          float* __restrict__ sh, int row, int wr, int D,
                                          int nv, float eps) {
  const int lane = threadIdx.x & 63;
  const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * D);
  float4 v[V > 0 ? V : 1];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < (V > 0 ? V : nv); ++i) {
    const float4 a = xr[lane + 64 * i];
    if constexpr (V > 0) v[i] = a;
    s += (a.x + a.y) + (a.z + a.w);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += xor_lane(s, o);
  const float mean = s * (1.0f / (float)D);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < (V > 0 ? V : nv); ++i) {
    const float4 a = V > 0 ? v[i] : xr[lane + 64 * i];
    const float b0 = a.x - mean, b1 = a.y - mean, b2 = a.z - mean, b3 = a.w - mean;
    q += (b0 * b0 + b1 * b1) + (b2 * b2 + b3 * b3);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) q += xor_lane(q, o);
  const float rstd = 1.0f / sqrtf(q * (1.0f / (float)D) + eps);
  const int sg = seg_of(segs, row);
  const float4* shift = reinterpret_cast<const float4*>(mod + (size_t)sg * 3 * D);
  const float4* scale = shift + D / 4;
  auto hval = [&](int i) -> float4 {
    const int c = lane + 64 * i;
    const float4 a = V > 0 ? v[i] : xr[c];
    const float4 shv = shift[c], sc = scale[c];
    return make_float4((1.0f + sc.x) * ((a.x - mean) * rstd) + shv.x,
                       (1.0f + sc.y) * ((a.y - mean) * rstd) + shv.y,
                       (1.0f + sc.z) * ((a.z - mean) * rstd) + shv.z,
                       (1.0f + sc.w) * ((a.w - mean) * rstd) + shv.w);
  };
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < (V > 0 ? V : nv); ++i) {
    const float4 h = hval(i);
    if constexpr (V > 0) v[i] = h;
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(h.x), fabsf(h.y)), fmaxf(fabsf(h.z), fabsf(h.w))));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, xor_lane(amax, o));
  float mult, rscale;
  e4m3_row_scale(amax, mult, rscale);
#pragma unroll
  for (int i = 0; i < (V > 0 ? V : nv); ++i) {
    const float4 h = V > 0 ? v[i] : hval(i);
    *reinterpret_cast<uint32_t*>(h8 + packed8_index(wr, 4 * (lane + 64 * i), D)) =
        e4m3x4(h.x, h.y, h.z, h.w, mult);
  }
  if (lane == 0) sh[wr] = rscale;
}

template <int V>
__global__ __launch_bounds__(256) void k_ln_modulate_f8(
    const float* __restrict__ x, const float* __restrict__ mod, SegTable segs, RowGroups rg,
    uint8_t* __restrict__ h8, float* __restrict__ sh, int rows, int D, float eps) {
  const int wr = blockIdx.x * 4 + (threadIdx.x >> 6);   // workspace row
  if (wr >= rows) return;
  const RowMap g = row_map(rg, wr);
  if (!g.live(wr)) return;
  ln_row_f8<V>(x, mod, segs, h8, sh, g.token(wr), wr, D, D / 256, eps);
}

hipError_t launch_ln_modulate_f8(const BlockShape& bs, const float* x, const float* mod,
                                 const SegTableHost& segs, void* h8, float* sh, float eps,
                                 hipStream_t s) {
  SegTable st;
  for (int i = 0; i < kMaxSegs; ++i) st.start[i] = segs.start[i];
  st.n = segs.n;
  if (!rows_valid(bs)) return hipErrorInvalidValue;
  // one group stops at its last token; several cover every workspace row
  const int rows = bs.rg.n == 1 ? bs.rg.ws_start[0] + bs.rg.count[0] : bs.rows;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  if (blocks == 0) return hipSuccess;
  uint8_t* out = static_cast<uint8_t*>(h8);
  if (bs.D == 3072)
    hipLaunchKernelGGL(k_ln_modulate_f8<12>, dim3(blocks), dim3(256), 0, s, x, mod, st, bs.rg, out,
                       sh, rows, bs.D, eps);
  else
    hipLaunchKernelGGL(k_ln_modulate_f8<0>, dim3(blocks), dim3(256), 0, s, x, mod, st, bs.rg, out,
                       sh, rows, bs.D, eps);
  return hipGetLastError();
}

hipError_t launch_ln_modulate(const BlockShape& bs, const float* x,
                              const float* mod, const SegTableHost& segs,
                              void* h, float eps, hipStream_t s) {
  SegTable st;
  for (int i = 0; i < kMaxSegs; ++i) st.start[i] = segs.start[i];
  st.n = segs.n;
  if (!rows_valid(bs)) return hipErrorInvalidValue;
  // one group stops at its last token; several cover every workspace row
  const int rows = bs.rg.n == 1 ? bs.rg.ws_start[0] + bs.rg.count[0] : bs.rows;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  if (blocks == 0) return hipSuccess;
  if (bs.D == 3072) {
    hipLaunchKernelGGL(k_ln_modulate<3072>, dim3(blocks), dim3(256), 0, s, x,
                       mod, st, bs.rg, reinterpret_cast<bf16*>(h), rows, eps);
  } else {
    hipLaunchKernelGGL(k_ln_modulate_any, dim3(blocks), dim3(256), 0, s, x,
                       mod, st, bs.rg, reinterpret_cast<bf16*>(h), rows, bs.D, eps);
  }
  return hipGetLastError();
}

}  // namespace flux3
