// K2 and K4: the block's two bf16 MFMA GEMMs with fused epilogues.
//
// The block listing of the Diffusers release post (everytik.com
// translation) runs attention and the SwiGLU MLP in parallel on the same
// modulated input h and adds their sum, times the gate, to the residual;
// "Inside the transformer" (rohitghumare.com guide) repeats it.  That
// structure gives two GEMMs per block:
//
//   K2  [q | k | v | gate | up] = h . [Wq; Wk; Wv; Wg; Wu]^T   (K = D)
//       epilogues: per-head RMSNorm + RoPE for q and k (head-major store),
//       v stored transposed for the attention kernel, silu(gate) * up.
//   K4  out = [o | act] . [Wo | Wd]^T                            (K = D + F)
//       epilogue: x += gate_s * out on the fp32 residual.
//
// Both operands are K-contiguous ("NT"): C[m][n] = sum_k A[m][k] * B[n][k],
// with B in torch Linear layout [out][in].  Tile 256 x 256 x 64, 4 waves in
// a 2 x 2 arrangement, each wave 128 x 128 = 4 x 4 blocks of the 32x32x16
// bf16 MFMA, fp32 accumulators.  A and B k-slices go global -> registers ->
// LDS (rows padded to 144 B so 16-byte fragment reads hit distinct banks),
// double-buffered with one barrier per k-step.  Workgroups are remapped so
// that the workgroups resident on one XCD (every 8th id) cover a compact
// group of C tiles and share A and B slices in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDK = BK + 8;               // padded LDS row, elements
constexpr int TILE_ELEMS = BM * LDK;      // one operand, one stage
constexpr int NTHREADS = 256;
constexpr int GROUP_M = 8;

struct Acc {
  f32x16 c[4][4];
};

// Tile coordinates for workgroup id b: XCD-major (ids b, b+8, ... share an
// XCD) and grouped GROUP_M M-tiles at a time within each XCD's range.
__device__ __forceinline__ void tile_coords(int b, int n_m, int n_n, int& mt,
                                            int& nt) {
  const int total = n_m * n_n;
  const int per = total / 8;
  const int lin = (b < per * 8) ? (b % 8) * per + b / 8 : b;
  const int group = GROUP_M * n_n;
  const int g = lin / group;
  const int first_m = g * GROUP_M;
  const int gm = min(n_m - first_m, GROUP_M);
  const int in = lin - g * group;
  mt = first_m + in % gm;
  nt = in / gm;
}

__device__ __forceinline__ void load_slices(u32x4 (&ra)[8], u32x4 (&rb)[8],
                                            const bf16* ap, size_t a_run,
                                            const bf16* const (&bp)[8], int ka,
                                            int kb) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    ra[i] = *reinterpret_cast<const u32x4*>(ap + i * a_run + ka);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    rb[i] = *reinterpret_cast<const u32x4*>(bp[i] + kb);
}

__device__ __forceinline__ void store_slices(bf16* As, bf16* Bs,
                                             const u32x4 (&ra)[8],
                                             const u32x4 (&rb)[8], int t) {
  const int row = t >> 3, ch = t & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<u32x4*>(As + (row + 32 * i) * LDK + ch * 8) = ra[i];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<u32x4*>(Bs + (row + 32 * i) * LDK + ch * 8) = rb[i];
}

__device__ __forceinline__ void mma_slice(const bf16* As, const bf16* Bs,
                                          Acc& acc, int wm, int wn,
                                          int lane) {
  const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(
          As + (wm * 128 + i * 32 + r) * LDK + kk * 16 + kh);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(
          Bs + (wn * 128 + j * 32 + r) * LDK + kk * 16 + kh);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc.c[i][j] = mfma32(a[i], b[j], acc.c[i][j]);
  }
}

// Main loop over k.  Phase 0 covers k tiles [0, nk0) with B pointers bp0,
// phase 1 (if nk1 > 0) the next nk1 tiles with bp1; A runs straight through.
__device__ __forceinline__ void gemm_mainloop(
    bf16* smem, Acc& acc, const bf16* ap, size_t a_run,
    const bf16* const (&bp0)[8], int nk0, const bf16* const (&bp1)[8],
    int nk1, int t) {
  const int wave = t >> 6, lane = t & 63;
  const int wm = wave >> 1, wn = wave & 1;
  bf16* As[2] = {smem, smem + TILE_ELEMS};
  bf16* Bs[2] = {smem + 2 * TILE_ELEMS, smem + 3 * TILE_ELEMS};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc.c[i][j][e] = 0.f;

  const int nk = nk0 + nk1;
  u32x4 ra[8], rb[8];
  load_slices(ra, rb, ap, a_run, bp0, 0, 0);
  store_slices(As[0], Bs[0], ra, rb, t);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const int nx = kt + 1;
    if (nx < nk) {
      if (nx < nk0)
        load_slices(ra, rb, ap, a_run, bp0, nx * BK, nx * BK);
      else
        load_slices(ra, rb, ap, a_run, bp1, nx * BK, (nx - nk0) * BK);
    }
    mma_slice(As[cur], Bs[cur], acc, wm, wn, lane);
    if (nx < nk) store_slices(As[cur ^ 1], Bs[cur ^ 1], ra, rb, t);
    __syncthreads();
  }
}

struct ProjArgs {
  const bf16* h;
  const bf16 *wq, *wk, *wv, *wg, *wu;
  const float *qn, *kn;
  const float2* rope;
  bf16 *q, *k, *vt, *cat;
  int M, n_pad, D, H, F;
  float eps;
};

// Position of token m inside a 16-key group of the transposed value store:
// groups of 4 keys are kept in the order 0, 2, 1, 3 so the attention
// kernel's 16-byte fragment reads line up with its probability layout.
__device__ __forceinline__ int vt_pos(int m) {
  const int g = (m >> 2) & 3;
  const int gp = ((g & 1) << 1) | (g >> 1);
  return (m & ~15) | (gp << 2) | (m & 3);
}

__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_proj(ProjArgs p) {
  __shared__ bf16 smem[4 * TILE_ELEMS];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int qkv_tiles = p.H / 2;
  const int n_n = 3 * qkv_tiles + p.F / 128;
  const int n_m = p.n_pad / BM;
  int mt, nt;
  tile_coords(blockIdx.x, n_m, n_n, mt, nt);
  const int m0 = mt * BM;

  int kind, head0 = 0, hid0 = 0;
  if (nt < 3 * qkv_tiles) {
    kind = nt / qkv_tiles;
    head0 = 2 * (nt % qkv_tiles);
  } else {
    kind = 3;
    hid0 = (nt - 3 * qkv_tiles) * 128;
  }
  const int D = p.D;
  const int row = t >> 3, ch = t & 7;
  const bf16* bp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bf16* W;
    int brow;
    if (kind < 3) {
      W = kind == 0 ? p.wq : (kind == 1 ? p.wk : p.wv);
      brow = head0 * 128 + 32 * i + row;
    } else {
      const int half = i >> 2, blk = i & 3;
      W = blk < 2 ? p.wg : p.wu;
      brow = hid0 + 64 * half + 32 * (blk & 1) + row;
    }
    bp[i] = W + (size_t)brow * D + ch * 8;
  }
  const bf16* ap = p.h + (size_t)(m0 + row) * D + ch * 8;
  Acc acc;
  gemm_mainloop(smem, acc, ap, (size_t)32 * D, bp, D / BK, bp, 0, t);

  const int r32 = lane & 31, hi = lane >> 5;
  if (kind < 2) {
    // per-head RMSNorm + RoPE; this wave holds one full head of 128 tokens
    const int head = head0 + wn;
    const float* nw = kind == 0 ? p.qn : p.kn;
    bf16* dst = (kind == 0 ? p.q : p.k) + (size_t)head * p.n_pad * kHeadDim;
    float w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = nw[j * 32 + r32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) ss += acc.c[i][j][e] * acc.c[i][j][e];
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) ss += xor_lane(ss, o);
        const float rs = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + p.eps);
        const bool live = m < p.M;
        const float2* rr = p.rope + (size_t)(live ? m : 0) * kRopePairs;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = j * 32 + r32;
          const float v = acc.c[i][j][e] * rs * w[j];
          const float vp = xor_lane(v, 1);
          const float2 cs = rr[d >> 1];
          const float o = (d & 1) ? (vp * cs.y + v * cs.x) : (v * cs.x - vp * cs.y);
          dst[(size_t)m * kHeadDim + d] = f2bf(live ? o : 0.f);
        }
      }
    }
  } else if (kind == 2) {
    // values, transposed: vt[head][d][pos(m)], 4 consecutive tokens per store
    const int head = head0 + wn;
    bf16* dst = p.vt + (size_t)head * kHeadDim * p.n_pad;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int mb = m0 + wm * 128 + i * 32 + 8 * g + 4 * hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = j * 32 + r32;
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = f2bf(mb + e < p.M ? acc.c[i][j][4 * g + e] : 0.f);
          *reinterpret_cast<bf16x4*>(dst + (size_t)d * p.n_pad + vt_pos(mb)) = v;
        }
      }
    }
  } else {
    // SwiGLU: blocks 0,1 are gate columns, blocks 2,3 the matching up columns
    const int ldc = D + p.F;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
        const bool live = m < p.M;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int hc = hid0 + 64 * wn + 32 * j + r32;
          const float g = acc.c[i][j][e], u = acc.c[i][j + 2][e];
          const float a = g / (1.0f + __expf(-g)) * u;
          p.cat[(size_t)m * ldc + D + hc] = f2bf(live ? a : 0.f);
        }
      }
    }
  }
}

struct OutArgs {
  const bf16* cat;
  const bf16 *wo, *wd;
  float* x;
  const float* mod;
  SegTable segs;
  int M, n_pad, D, F;
};

__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_out(OutArgs p) {
  __shared__ bf16 smem[4 * TILE_ELEMS];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int D = p.D, F = p.F;
  const int n_n = D / BN;
  const int n_m = p.n_pad / BM;
  int mt, nt;
  tile_coords(blockIdx.x, n_m, n_n, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int row = t >> 3, ch = t & 7;
  const bf16 *bp0[8], *bp1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bp0[i] = p.wo + (size_t)(n0 + 32 * i + row) * D + ch * 8;
    bp1[i] = p.wd + (size_t)(n0 + 32 * i + row) * F + ch * 8;
  }
  const int ldc = D + F;
  const bf16* ap = p.cat + (size_t)(m0 + row) * ldc + ch * 8;
  Acc acc;
  gemm_mainloop(smem, acc, ap, (size_t)32 * ldc, bp0, D / BK, bp1, F / BK, t);

  const int r32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
      if (m >= p.M) continue;
      const float* gate = p.mod + (size_t)seg_of(p.segs, m) * 3 * D + 2 * D;
      float* xr = p.x + (size_t)m * D;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 128 + j * 32 + r32;
        xr[n] += gate[n] * acc.c[i][j][e];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_proj(const BlockShape& bs, const BlockWeightsDev& w,
                            const float* rope, const WsPtrs& ws, float eps,
                            hipStream_t s) {
  ProjArgs p;
  p.h = static_cast<const bf16*>(ws.h);
  p.wq = static_cast<const bf16*>(w.wq);
  p.wk = static_cast<const bf16*>(w.wk);
  p.wv = static_cast<const bf16*>(w.wv);
  p.wg = static_cast<const bf16*>(w.w_gate);
  p.wu = static_cast<const bf16*>(w.w_up);
  p.qn = w.q_norm;
  p.kn = w.k_norm;
  p.rope = reinterpret_cast<const float2*>(rope);
  p.q = static_cast<bf16*>(ws.q);
  p.k = static_cast<bf16*>(ws.k);
  p.vt = static_cast<bf16*>(ws.vt);
  p.cat = static_cast<bf16*>(ws.cat);
  p.M = bs.M;
  p.n_pad = bs.n_pad;
  p.D = bs.D;
  p.H = bs.H;
  p.F = bs.F;
  p.eps = eps;
  const int n_n = 3 * (bs.H / 2) + bs.F / 128;
  const int n_m = bs.n_pad / BM;
  hipLaunchKernelGGL(k_gemm_proj, dim3(n_m * n_n), dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm_out(const BlockShape& bs, const BlockWeightsDev& w,
                           const WsPtrs& ws, float* x, const float* mod,
                           const SegTableHost& segs, hipStream_t s) {
  OutArgs p;
  p.cat = static_cast<const bf16*>(ws.cat);
  p.wo = static_cast<const bf16*>(w.wo);
  p.wd = static_cast<const bf16*>(w.w_down);
  p.x = x;
  p.mod = mod;
  for (int i = 0; i < kMaxSegs; ++i) p.segs.start[i] = segs.start[i];
  p.segs.n = segs.n;
  p.M = bs.M;
  p.n_pad = bs.n_pad;
  p.D = bs.D;
  p.F = bs.F;
  const int n_n = bs.D / BN;
  const int n_m = bs.n_pad / BM;
  hipLaunchKernelGGL(k_gemm_out, dim3(n_m * n_n), dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace flux3
