// The denoise loop's per-step update ("The denoise loop", rohitghumare.com
// guide; the preview step of the Diffusers release post, 15jq.com):
//   x0 preview = latent - sigma * v          (the current guess of the image)
//   latent    += (sigma_next - sigma) * v    (flow-matching Euler step)
// over the noisy image's latent tokens, fp32.  HBM-bound: 8 B read and 4 B
// written per element (plus 4 B for the preview).
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

__global__ __launch_bounds__(256) void k_euler(const float4* __restrict__ v,
                                               float4* __restrict__ latent,
                                               float4* __restrict__ x0, int64_t n4,
                                               float sigma, float step) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 d = v[i];
  float4 x = latent[i];
  if (x0) {
    float4 p;
    p.x = x.x - sigma * d.x;
    p.y = x.y - sigma * d.y;
    p.z = x.z - sigma * d.z;
    p.w = x.w - sigma * d.w;
    x0[i] = p;
  }
  x.x += step * d.x;
  x.y += step * d.y;
  x.z += step * d.z;
  x.w += step * d.w;
  latent[i] = x;
}

}  // namespace

hipError_t launch_euler(const float* v, float* latent, float* x0, int64_t n, float sigma,
                        float sigma_next, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_euler, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(v), reinterpret_cast<float4*>(latent),
                     reinterpret_cast<float4*>(x0), n4, sigma, sigma_next - sigma);
  return hipGetLastError();
}

}  // namespace flux3
