// Modulation vectors from timesteps, on the device.
//
// The adaLN modulation of a block comes from the timestep ("Speed,
// architecture, and how the tokens move", 15jq.com post: image tokens take
// the current timestep, text and reference tokens t = 0; "What step
// distillation removed", rohitghumare.com guide: a 256 -> 3072 -> 3072
// embedder with no biases, and for the distilled flow map a second embedder
// of the target timestep whose output is added).  With e(t) the 256-d
// sinusoidal embedding of tau = 1000 t (cosines first, frequencies
// 10000^(-i/128)), E(t) = W2 silu(W1 e(t)) and
//   mod_mode = W_mod[mode] silu(E(t_mode) [+ E'(t_target)])
// split into shift, scale and gate.
//
// All of it is matrix-vector work over bf16 weights (about 190 MB per
// stage at width 3072), so it is bound by HBM: one pass over each weight
// matrix serves every timestep that uses it.  fp32 accumulation, fp64 for
// the sinusoids.
#include <string.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

constexpr int kEmbed = 256;          // sinusoidal embedding width
constexpr int kMaxRowsPerWave = 16;
constexpr int kTargetWaves = 2048;   // 8 waves on each of 256 CUs
constexpr int kMaxVec = 3;           // vectors sharing one pass over W
constexpr int kMaxChunks = 8;        // 512-value chunks of a row (K <= 4096)

struct Timesteps {
  float t[4];
  int n;
};

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

// e(t_j) for each timestep: [cos(tau f_i), sin(tau f_i)], i < 128, in fp64.
__global__ __launch_bounds__(128) void k_timestep_embed(Timesteps ts, float* __restrict__ emb) {
  const int j = blockIdx.x, i = threadIdx.x;
  if (j >= ts.n) return;
  const double tau = 1000.0 * (double)ts.t[j];
  const double f = pow(10000.0, -(double)i / 128.0);
  emb[j * kEmbed + i] = (float)cos(tau * f);
  emb[j * kEmbed + 128 + i] = (float)sin(tau * f);
}

// v from the lane the DPP control selects (0 where the row is masked off).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes with DPP row operations (no LDS round trips): pairs,
// quads, half rows, rows, then rows 0+1 and 2+3 into rows 1 and 3, and rows
// 0..2 into row 3; lane 63 ends with the total.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);          // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);          // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);         // row_half_mirror
  v += dpp<0x140>(v);         // row_mirror
  v += dpp<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
  v += dpp<0x143, 0xC>(v);    // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// One matrix of a fused matrix-vector launch: y_v = W act(x_v + x_add) for
// nv input vectors, written to y + y_off + v * y_stride and, for a one-vector
// job, also to the extra destinations (segments sharing a mode).
struct GemvJob {
  const bf16* w;        // [rows][K], row-major
  int rows;
  int nv;               // input vectors
  int x_off;            // first input vector (float offset into x)
  int x_add_off;        // vector added to every input before the activation, or -1
  int y_off, y_stride;
  int ndst;             // extra destinations (float offsets into y), <= kMaxSegs
  int dst[kMaxSegs];
};

constexpr int kMaxJobs = 3;

struct GemvArgs {
  GemvJob job[kMaxJobs];
  int njobs;
  int block0[kMaxJobs + 1];   // first workgroup of each job
  int K;
  const float* x;       // input vectors, stride K
  int silu_in;          // apply silu to (x + x_add) as it is read
  int rows_per_wave;
  float* y;
};

// Fused matrix-vector products.  Lane l always covers the k-values
// [8 l + 512 c, 8 l + 512 c + 8) of a row (c < K / 512), so it keeps its
// part of the input vectors in registers (with the activation applied) and
// needs no LDS.  A wave streams rows_per_wave consecutive rows of one job
// two at a time, the next two rows' 16-byte loads in flight (one
// instruction reads 1 KiB of a row) while the current ones are summed
// across the wave with DPP.
template <int NV, int NC>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs p) {
  static_assert(NV >= 1 && NV <= kMaxVec && NC >= 1 && NC <= kMaxChunks, "gemv shape");
  int jb = 0;
  while (jb + 1 < p.njobs && (int)blockIdx.x >= p.block0[jb + 1]) ++jb;
  const GemvJob& J = p.job[jb];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int K = p.K;
  const int r_begin = ((blockIdx.x - p.block0[jb]) * 4 + wave) * p.rows_per_wave;
  const int r_end = min(r_begin + p.rows_per_wave, J.rows);
  if (r_begin >= J.rows) return;

  // this lane's k-values of the input vectors: two 16-byte loads per chunk,
  // all issued before any is used; then the optional added vector; then the
  // activation
  float xr[NV][NC][8];
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int k0 = lane * 8 + c * 512;
      f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = lo;
      if (v < J.nv && k0 < K) {
        const f32x4* px = reinterpret_cast<const f32x4*>(p.x + (size_t)J.x_off + (size_t)v * K + k0);
        lo = px[0];
        hi = px[1];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xr[v][c][e] = lo[e];
        xr[v][c][4 + e] = hi[e];
      }
    }
  if (J.x_add_off >= 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int k0 = lane * 8 + c * 512;
      if (k0 >= K) break;
      const f32x4* pa = reinterpret_cast<const f32x4*>(p.x + (size_t)J.x_add_off + k0);
      const f32x4 lo = pa[0], hi = pa[1];
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xr[v][c][e] += lo[e];
          xr[v][c][4 + e] += hi[e];
        }
    }
  }
  if (p.silu_in) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) xr[v][c][e] = silu(xr[v][c][e]);
  }

  // Loads are unconditional (so none waits on another): a row past the end
  // re-reads the last row and a chunk past K re-reads the last chunk; those
  // values meet zero inputs or are never stored.
  auto load = [&](bf16x8 (&buf)[2][NC], int row) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int rr = min(row + q, r_end - 1);
        const int k0 = min(lane * 8 + c * 512, K - 8);
        buf[q][c] = *reinterpret_cast<const bf16x8*>(J.w + (size_t)rr * K + k0);
      }
  };
  auto finish = [&](const bf16x8 (&buf)[2][NC], int row) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (row + q >= r_end) break;
      float acc[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (lane * 8 + c * 512 >= K) break;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float we = bf2f(buf[q][c][e]);
#pragma unroll
          for (int v = 0; v < NV; ++v) acc[v] = __builtin_fmaf(we, xr[v][c][e], acc[v]);
        }
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        if (v >= J.nv) break;
        const float sum = wave_sum(acc[v]);
        if (lane == 0) {
          p.y[(size_t)J.y_off + (size_t)v * J.y_stride + row + q] = sum;
          if (v == 0)
            for (int d = 0; d < J.ndst; ++d) p.y[(size_t)J.dst[d] + row + q] = sum;
        }
      }
    }
  };
  bf16x8 b0[2][NC], b1[2][NC];
  load(b0, r_begin);
  for (int row = r_begin; row < r_end; row += 4) {
    load(b1, row + 2);
    finish(b0, row);
    if (row + 2 >= r_end) break;
    load(b0, row + 4);
    finish(b1, row + 2);
  }
}

GemvJob job(const void* w, int rows, int nv, int x_off, int y_off, int y_stride) {
  GemvJob j;
  j.w = static_cast<const bf16*>(w);
  j.rows = rows;
  j.nv = nv;
  j.x_off = x_off;
  j.x_add_off = -1;
  j.y_off = y_off;
  j.y_stride = y_stride;
  j.ndst = 0;
  return j;
}

hipError_t launch_gemv(GemvArgs& p, int njobs, int K, int max_nv, hipStream_t s) {
  p.njobs = njobs;
  p.K = K;
  // about kTargetWaves waves in all, at most kMaxRowsPerWave rows each
  int rows = 0;
  for (int j = 0; j < njobs; ++j) rows += p.job[j].rows;
  p.rows_per_wave = std::min(kMaxRowsPerWave, std::max(1, (rows + kTargetWaves - 1) / kTargetWaves));
  const int rows_per_block = 4 * p.rows_per_wave;
  int blocks = 0;
  for (int j = 0; j < njobs; ++j) {
    p.block0[j] = blocks;
    blocks += (p.job[j].rows + rows_per_block - 1) / rows_per_block;
  }
  p.block0[njobs] = blocks;
  // instantiate for the vectors and 512-value chunks in use
  const int nc = (K + 511) / 512;
  const dim3 g(blocks), b(256);
#define FLUX3_GEMV_NC(NV)                                                          \
  if (nc <= 1) hipLaunchKernelGGL((k_gemv<NV, 1>), g, b, 0, s, p);                 \
  else if (nc <= 2) hipLaunchKernelGGL((k_gemv<NV, 2>), g, b, 0, s, p);            \
  else if (nc <= 4) hipLaunchKernelGGL((k_gemv<NV, 4>), g, b, 0, s, p);            \
  else if (nc <= 6) hipLaunchKernelGGL((k_gemv<NV, 6>), g, b, 0, s, p);            \
  else hipLaunchKernelGGL((k_gemv<NV, 8>), g, b, 0, s, p);
  if (max_nv <= 1) {
    FLUX3_GEMV_NC(1)
  } else if (max_nv == 2) {
    FLUX3_GEMV_NC(2)
  } else {
    FLUX3_GEMV_NC(3)
  }
#undef FLUX3_GEMV_NC
  return hipGetLastError();
}

}  // namespace

size_t modulation_workspace_floats(int D) {
  // embeddings [4][256], hidden vectors [4][D], E [4][D]
  return 4 * (size_t)kEmbed + 8 * (size_t)D;
}

// Four launches: the embeddings, then the first embedder layer (and the
// target embedder's), the second layer (and the target's), and the
// modulation linear of every used mode on silu(E + E'), written to all
// segments of that mode.  Workspace: emb [4][256], a1 [4][D] (hidden
// vectors), e [4][D] (E per timestep, E' of the target last).
hipError_t launch_modulation(const ModulationShape& ms, const ModulationWeightsDev& w,
                             const SegTableHost& segs, const int32_t* seg_mode, float* mod,
                             float* ws, hipStream_t s, float* final_mod) {
  const int D = ms.D;
  const int nt = ms.n_t;
  float* emb = ws;                        // [4][256]
  float* a1 = ws + 4 * kEmbed;            // [4][D]
  float* e = a1 + 4 * (size_t)D;          // [4][D]
  Timesteps ts;
  ts.n = nt + (ms.has_target ? 1 : 0);    // the target timestep last
  for (int j = 0; j < 4; ++j) ts.t[j] = j < ts.n ? ms.t[j] : 0.f;
  hipLaunchKernelGGL(k_timestep_embed, dim3(ts.n), dim3(128), 0, s, ts, emb);
  hipError_t r = hipGetLastError();
  if (r != hipSuccess) return r;
  GemvArgs p;
  memset(&p, 0, sizeof p);
  // a1[j] = W1 e(t_j); a1[nt] = W1' e(t_target)
  p.silu_in = 0;
  p.x = emb;
  p.y = a1;
  p.job[0] = job(w.w1, D, nt, 0, 0, D);
  int nj = 1;
  if (ms.has_target) p.job[nj++] = job(w.w1_tgt, D, 1, nt * kEmbed, nt * D, D);
  if ((r = launch_gemv(p, nj, kEmbed, nt, s)) != hipSuccess) return r;
  // e[j] = W2 silu(a1[j]); e[nt] = W2' silu(a1[nt])
  p.silu_in = 1;
  p.x = a1;
  p.y = e;
  p.job[0] = job(w.w2, D, nt, 0, 0, D);
  nj = 1;
  if (ms.has_target) p.job[nj++] = job(w.w2_tgt, D, 1, nt * D, nt * D, D);
  if ((r = launch_gemv(p, nj, D, nt, s)) != hipSuccess) return r;
  // mod[segment] = W_mod[mode] silu(e[t_index[mode]] + e[nt])
  p.x = e;
  p.y = mod;
  nj = 0;
  for (int m = 0; m < 3; ++m) {
    GemvJob jb = job(w.w_mod[m], 3 * D, 0, ms.t_index[m] * D, 0, 0);
    jb.x_add_off = ms.has_target ? nt * D : -1;
    for (int sg = 0; sg < segs.n; ++sg) {
      if (seg_mode[sg] != m) continue;
      if (jb.nv == 0) {
        jb.nv = 1;
        jb.y_off = sg * 3 * D;
      } else {
        jb.dst[jb.ndst++] = sg * 3 * D;
      }
    }
    if (jb.nv) p.job[nj++] = jb;
  }
  if ((r = launch_gemv(p, nj, D, 1, s)) != hipSuccess) return r;
  if (!final_mod) return hipSuccess;
  // output layer: final_mod = W_final silu(e[t_index[image]] + e[nt]), 2 D rows
  p.y = final_mod;
  p.job[0] = job(w.w_final, 2 * D, 1, ms.t_index[1] * D, 0, 0);
  p.job[0].x_add_off = ms.has_target ? nt * D : -1;
  return launch_gemv(p, 1, D, 1, s);
}

}  // namespace flux3
