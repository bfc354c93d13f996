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
// bf16 MFMA, fp32 accumulators.  A and B k-slices stream from global memory
// straight into LDS (gfx950 global_load_lds_dwordx4, no staging registers),
// XOR-swizzled instead of padded, double-buffered with one barrier per
// k-step; fragment reads and the next slice's loads are interleaved with
// the MFMAs.  Workgroups are remapped so that the workgroups resident on one
// XCD (every 8th id) cover a compact group of C tiles and share A and B
// slices in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int ROW_BYTES = BK * 2;             // one tile row of a k-slice
constexpr int OP_BYTES = BM * ROW_BYTES;      // one operand, one stage: 32 KiB
constexpr int STAGE_BYTES = 2 * OP_BYTES;     // A then B
constexpr int LDS_BYTES = 2 * STAGE_BYTES;    // double-buffered: 128 KiB
constexpr int NTHREADS = 256;
constexpr int GROUP_M = 8;

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gvoid;

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

// Where this wave's share of one operand tile comes from: wave w loads tile
// rows [64w, 64w + 64), i.e. the 32-row runs 2w (lo) and 2w + 1 (hi); each
// run has a wave-uniform base pointer (its first row at k = 0) and all rows
// share the stride ld.
struct Src {
  const bf16* lo;
  const bf16* hi;
  int ld;
};

// LDS layout of a k-slice: row r of the tile occupies 128 contiguous bytes
// (no padding); its 16-byte chunk c sits in slot c ^ ((r / 2) % 8).  With
// 64 banks this keeps the MFMA fragment reads (32 consecutive rows, one
// chunk, per half-wave) conflict-free, and it lets each wave fill whole
// 1-KiB blocks with direct global->LDS loads: lane l of a block writes slot
// l % 8 of row l / 8 and therefore fetches chunk (l % 8) ^ swizzle(row).
__device__ __forceinline__ void issue_operand(const Src& S, int k, lds_u8* dst,
                                              int wave, int lane) {
  const int rsub = lane >> 3, slot = lane & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = slot ^ ((4 * (i & 1) + (lane >> 4)) & 7);   // (row/2)%8 of this row
    const bf16* g = (i < 4 ? S.lo : S.hi) + (8 * (i & 3) + rsub) * S.ld + k + c * 8;
    __builtin_amdgcn_global_load_lds((gvoid*)g, (lds_void*)(dst + (64 * wave + 8 * i) * ROW_BYTES),
                                     16, 0, 0);
  }
}

__device__ __forceinline__ void wait_loads() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
}

struct Frags {
  bf16x8 a[4], b[4];
};

__device__ __forceinline__ void read_frags(Frags& f, const lds_u8* As, const lds_u8* Bs,
                                           int wm, int wn, int lane, int kk) {
  const int r = lane & 31;
  const int chunk = ((2 * kk + (lane >> 5)) ^ ((lane >> 1) & 7)) << 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.a[i] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
        As + (wm * 128 + i * 32 + r) * ROW_BYTES + chunk);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.b[j] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
        Bs + (wn * 128 + j * 32 + r) * ROW_BYTES + chunk);
}

__device__ __forceinline__ void mma_frags(const Frags& f, Acc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.c[i][j] = mfma32(f.a[i], f.b[j], acc.c[i][j]);
}

// Scheduling-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMFMA = 0x008;
constexpr int kSchedVMEMRead = 0x020;
constexpr int kSchedDSRead = 0x100;

// One BK slice.  The 8 fragment reads of k-step kk+1 are interleaved one by
// one with the MFMAs of k-step kk; with_loads also spreads the next slice's
// 16 direct loads over the second half of k-steps 0 and 1.
template <bool with_loads>
__device__ __forceinline__ void mma_slice(const lds_u8* As, const lds_u8* Bs,
                                          Acc& acc, int wm, int wn, int lane) {
  Frags f0, f1;
  read_frags(f0, As, Bs, wm, wn, lane, 0);
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    Frags& cur = (kk & 1) ? f1 : f0;
    Frags& nxt = (kk & 1) ? f0 : f1;
    if (kk + 1 < BK / 16) read_frags(nxt, As, Bs, wm, wn, lane, kk + 1);
    mma_frags(cur, acc);
    if (kk + 1 < BK / 16) {
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
      }
      if (with_loads && kk < 2) {
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedVMEMRead, 1, 0);
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 8, 0);
      }
    }
  }
}

// Main loop over k.  Phase 0 covers k tiles [0, nk0) with B rows from B0,
// phase 1 (if nk1 > 0) the next nk1 tiles from B1; A runs straight through.
// Slice kt+1 streams into the other LDS buffer while slice kt is consumed.
__device__ __forceinline__ void gemm_mainloop(lds_u8* smem, Acc& acc, const Src& A,
                                              const Src& B0, int nk0, const Src& B1,
                                              int nk1) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc.c[i][j][e] = 0.f;

  const int nk = nk0 + nk1;
  issue_operand(A, 0, smem, wave, lane);
  issue_operand(B0, 0, smem + OP_BYTES, wave, lane);
  wait_loads();
  __syncthreads();
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int cur = (kt & 1) * STAGE_BYTES;
    const int nxt = STAGE_BYTES - cur;
    const int kn = kt + 1;
    const bool ph0 = kn < nk0;
    issue_operand(A, kn * BK, smem + nxt, wave, lane);
    issue_operand(ph0 ? B0 : B1, ph0 ? kn * BK : (kn - nk0) * BK, smem + nxt + OP_BYTES, wave,
                  lane);
    mma_slice<true>(smem + cur, smem + cur + OP_BYTES, acc, wm, wn, lane);
    wait_loads();
    __syncthreads();
  }
  const int last = ((nk - 1) & 1) * STAGE_BYTES;
  mma_slice<false>(smem + last, smem + last + OP_BYTES, acc, wm, wn, lane);
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
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[LDS_BYTES];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
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
  // first row of 32-row run i of the B tile
  auto b_run = [&](int i) -> const bf16* {
    if (kind < 3) {
      const bf16* W = kind == 0 ? p.wq : (kind == 1 ? p.wk : p.wv);
      return W + (size_t)(head0 * 128 + 32 * i) * D;
    }
    const int half = i >> 2, blk = i & 3;
    const bf16* W = blk < 2 ? p.wg : p.wu;
    return W + (size_t)(hid0 + 64 * half + 32 * (blk & 1)) * D;
  };
  Src A, B;
  A.lo = p.h + (size_t)(m0 + 64 * wave) * D;
  A.hi = A.lo + (size_t)32 * D;
  A.ld = D;
  B.lo = b_run(2 * wave);
  B.hi = b_run(2 * wave + 1);
  B.ld = D;
  Acc acc;
  gemm_mainloop(smem, acc, A, B, D / BK, B, 0);

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
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[LDS_BYTES];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int D = p.D, F = p.F;
  const int n_n = D / BN;
  const int n_m = p.n_pad / BM;
  int mt, nt;
  tile_coords(blockIdx.x, n_m, n_n, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int ldc = D + F;
  Src A, B0, B1;
  A.lo = p.cat + (size_t)(m0 + 64 * wave) * ldc;
  A.hi = A.lo + (size_t)32 * ldc;
  A.ld = ldc;
  B0.lo = p.wo + (size_t)(n0 + 64 * wave) * D;
  B0.hi = B0.lo + (size_t)32 * D;
  B0.ld = D;
  B1.lo = p.wd + (size_t)(n0 + 64 * wave) * F;
  B1.hi = B1.lo + (size_t)32 * F;
  B1.ld = F;
  Acc acc;
  gemm_mainloop(smem, acc, A, B0, D / BK, B1, F / BK);

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
