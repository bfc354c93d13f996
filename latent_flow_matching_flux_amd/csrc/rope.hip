// Rotary tables for a token layout (the pipeline's prepare_rope_inputs step).
//
// Positions follow the RoPE position table of the Diffusers release post
// (Chinese translation, everytik.com): text token i at (0, 0, 0, i); the
// noisy-image token at grid (row, col) at (0, row/2, col/2, 0); reference k
// at (0, row/2, col/2, -(k+1)) (negative l offset, ifeeling.app summary).
// Each 128-dim head gives each of the four axes (t, h, w, l) 32 dims
// ("Speed, architecture, and how the tokens move", 15jq.com post): pair
// p = 16a + j turns by pos[a] * theta^(-2j/32).  Angles and cos/sin are
// evaluated in fp64 and rounded once to fp32.
//
// One thread per (token, pair); output float2 (cos, sin) at [token][pair].
// HBM-bound: 8 bytes written per thread, no reads.
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

__global__ __launch_bounds__(256) void k_rope_tables(RopeLayoutDev lay,
                                                     float2* __restrict__ out,
                                                     int64_t n) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n * kRopePairs) return;
  const int64_t tok = gid >> 6;
  const int pair = (int)(gid & 63);
  const int axis = pair >> 4;
  const int j = pair & 15;

  // (t, h, w, l) of this token
  double pos[4] = {0.0, 0.0, 0.0, 0.0};
  int64_t r = tok;
  if (r < lay.n_text) {
    pos[3] = (double)r;
  } else {
    r -= lay.n_text;
    const int64_t n_img = (int64_t)lay.grid_h * lay.grid_w;
    if (r < n_img) {
      pos[1] = (double)(r / lay.grid_w) * lay.hw_scale;
      pos[2] = (double)(r % lay.grid_w) * lay.hw_scale;
    } else {
      r -= n_img;
      for (int k = 0; k < lay.n_refs; ++k) {
        const int64_t nk = (int64_t)lay.ref_h[k] * lay.ref_w[k];
        if (r < nk) {
          pos[1] = (double)(r / lay.ref_w[k]) * lay.hw_scale;
          pos[2] = (double)(r % lay.ref_w[k]) * lay.hw_scale;
          pos[3] = -(double)(k + 1);
          break;
        }
        r -= nk;
      }
    }
  }
  const double omega = pow(lay.theta, -2.0 * (double)j / 32.0);
  const double phi = pos[axis] * omega;
  out[gid] = make_float2((float)cos(phi), (float)sin(phi));
}

hipError_t launch_rope_tables(const RopeLayoutDev& lay, float* rope, int64_t n,
                              hipStream_t s) {
  const int64_t total = n * kRopePairs;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(k_rope_tables, dim3(blocks), dim3(256), 0, s, lay,
                     reinterpret_cast<float2*>(rope), n);
  return hipGetLastError();
}

}  // namespace flux3
