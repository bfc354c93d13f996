// K3: full bidirectional softmax attention, flash-style, for gfx950.
//
// Every token attends to every token of the call, with no mask ("Speed,
// architecture, and how the tokens move", 15jq.com post: everything attends
// to everything in the joint stage, each stream only to itself in the
// per-mode stage -- the per-mode case is this kernel on one stream's rows).
// Queries and keys arrive RMS-normalised and rotated; the scale is
// 1/sqrt(128).
//
// Work split: a workgroup is 4 waves x 64 queries of one head (one wave per
// SIMD).  A wave keeps its 64 queries in registers and computes
// S^T = K . Q^T with the 32x32x16 bf16 MFMA, so every lane owns one query of
// each 32-query block and 16 of each 32 keys; O^T = V^T . P^T then takes the
// probabilities straight from those registers as the B operand (V arrives
// transposed, keys permuted inside each group of 16 to match).  Every K or
// V^T fragment read from LDS feeds two MFMAs (one per 32-query block).
//
// K and V^T tiles of 64 keys stream from global memory straight into a
// 4-deep LDS ring (gfx950 direct loads, XOR-swizzled rows), two tiles ahead.
// Keys are processed in blocks of 32: the QK^T MFMAs of the next block are
// issued before the softmax of the current one.
//
// Online softmax with lazy rescaling: scores are kept in the log2 domain
// (log2(e)/sqrt(128) folded into the scale); the running reference max of a
// query only moves -- and O and the running sum are only rescaled -- when a
// tile's max exceeds it by more than TAU, so exp2(s - m) <= 2^TAU and fp32 /
// bf16 never overflow.  Keys past the sequence end are masked to -inf (the
// workspace pads them with zeros).
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

constexpr int QW = 64;                 // queries per wave
constexpr int WAVES = 4;
constexpr int AQ = QW * WAVES;         // queries per workgroup
constexpr int AKV = 64;                // keys per tile
constexpr int NSTAGE = 4;              // LDS ring depth (tiles)
constexpr int K_ROW = kHeadDim * 2;    // 256 B: one key of K
constexpr int V_ROW = AKV * 2;         // 128 B: one dim of V^T for the tile
constexpr int K_BYTES = AKV * K_ROW;   // 16 KiB
constexpr int V_BYTES = kHeadDim * V_ROW;  // 16 KiB
constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;  // 128 KiB
constexpr int DMA_PER_TILE = 8;        // per wave: 4 for K, 4 for V^T
constexpr float TAU = 8.0f;

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef const __attribute__((address_space(3))) bf16x8 lds_frag;

struct AttnArgs {
  const bf16 *q, *k, *vt;
  bf16* out;         // cat buffer, row stride ldo
  int M, n_pad, H, ldo;
  float scale_log2;  // log2(e) / sqrt(head_dim)
};

// Direct global->LDS load, 16 bytes per lane to LDS byte lds_off + 16 * lane
// (see the projection GEMM for why it is an asm statement).
__device__ __forceinline__ void dma16(const bf16* g, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_off)
               : "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// LDS layouts.  K tile: key r's 256 bytes, 16-byte chunk c in slot
// c ^ (r % 16).  V^T tile: dim r's 128 bytes, chunk c in slot c ^ ((r/2) % 8).
// Both keep 16 consecutive rows of a fragment read on distinct banks.
__device__ __forceinline__ void issue_tile(const bf16* kh, const bf16* vh, int n_pad, int kv0,
                                           uint32_t stage, int wave, int lane) {
  // K: this wave loads keys [16 wave, 16 wave + 16): 4 blocks of 4 rows x 256 B
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * wave + 4 * i + (lane >> 4);
    const int c = (lane & 15) ^ (row & 15);
    dma16(kh + (size_t)(kv0 + row) * kHeadDim + c * 8, stage + (16 * wave + 4 * i) * K_ROW);
  }
  // V^T: this wave loads dims [32 wave, 32 wave + 32): 4 blocks of 8 rows x 128 B
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    dma16(vh + (size_t)row * n_pad + kv0 + c * 8, stage + K_BYTES + (32 * wave + 8 * i) * V_ROW);
  }
}

typedef f32x16 SHalf[2];        // S^T for 32 keys x 2 query blocks
typedef bf16x8 PHalf[2][2];     // P^T fragments: [16-key half][query block]

// S^T for key block kb (32 keys) of a tile: 8 head-dim steps x 2 query blocks.
__device__ __forceinline__ void qk_half(SHalf& S, const lds_u8* Ks, int kb,
                                        const bf16x8 (&qf)[2][8], int lane) {
  const int r = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int e = 0; e < 16; ++e) S[qb][e] = 0.f;
  const int row = kb * 32 + r;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int c = (2 * ks + hh) ^ (row & 15);
    const bf16x8 a = *reinterpret_cast<lds_frag*>(Ks + row * K_ROW + c * 16);
    S[0] = mfma32(a, qf[0][ks], S[0]);
    S[1] = mfma32(a, qf[1][ks], S[1]);
  }
}

// O^T += V^T . P^T for key block kb (32 keys) of a tile.
__device__ __forceinline__ void pv_half(f32x16 (&o)[4][2], const lds_u8* Vs, int kb,
                                        const PHalf& pf, int lane) {
  const int r = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int row = d * 32 + r;
      const int c = (4 * kb + 2 * tt + hh) ^ ((row >> 1) & 7);
      const bf16x8 a = *reinterpret_cast<lds_frag*>(Vs + row * V_ROW + c * 16);
      o[d][0] = mfma32(a, pf[tt][0], o[d][0]);
      o[d][1] = mfma32(a, pf[tt][1], o[d][1]);
    }
}

// Softmax of one 32-key block: raw scores S (in units of q.k), masking keys
// past the end when MASK.  The reference max moves only when the block's
// max (log2 domain) exceeds it by more than TAU; then `alpha` is the factor
// that O must be multiplied by once the PV MFMAs issued so far have landed,
// and the function returns true.  P = exp2(scale * S - m) goes to bf16.
template <bool MASK>
__device__ __forceinline__ bool softmax_half(const SHalf& S, PHalf& pf, float (&m_ref)[2],
                                             float (&l_sum)[2], float (&alpha)[2], float scale,
                                             int key0, int M, int hh) {
  float mx[2];
  float v[2][16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      v[qb][e] = S[qb][e];
      if constexpr (MASK) {
        const int j = key0 + 8 * (e >> 2) + 4 * hh + (e & 3);
        v[qb][e] = j < M ? v[qb][e] : -INFINITY;
      }
    }
    float m = v[qb][0];
#pragma unroll
    for (int e = 1; e < 16; ++e) m = fmaxf(m, v[qb][e]);
    m *= scale;
    mx[qb] = fmaxf(m, xor_lane(m, 32));
  }
  // branch-free so the whole softmax stays one scheduling region with the
  // MFMAs it hides behind; alpha is 1 when nothing moved
  const bool grow = (mx[0] > m_ref[0] + TAU) || (mx[1] > m_ref[1] + TAU);
  const bool any = __any(grow);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float m_new = any ? fmaxf(m_ref[qb], mx[qb]) : m_ref[qb];
    alpha[qb] = __builtin_amdgcn_exp2f(m_ref[qb] - m_new);
    m_ref[qb] = m_new;
    l_sum[qb] *= alpha[qb];
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(v[qb][e], scale, -m_ref[qb]));
      l += pv;
      pf[e >> 3][qb][e & 7] = f2bf(pv);
    }
    l_sum[qb] += l;
  }
  return any;
}

__device__ __forceinline__ void rescale_o(f32x16 (&o)[4][2], const float (&alpha)[2]) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[d][qb][e] *= alpha[qb];
}

__global__ __launch_bounds__(256, 1) void k_attention(AttnArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[LDS_BYTES];
  lds_u8* smem = (lds_u8*)smem_raw;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int r32 = lane & 31, hh = lane >> 5;

  // workgroup -> (head, query block); the workgroups an XCD runs (every 8th
  // id) share heads so K and V stay in that XCD's L2
  const int nqb = (p.M + AQ - 1) / AQ;
  int head, qblk;
  if (p.H % 8 == 0) {
    const int b = blockIdx.x, xcd = b & 7, idx = b >> 3;
    const int hpx = p.H / 8;
    head = xcd * hpx + idx / nqb;
    qblk = idx % nqb;
  } else {
    head = blockIdx.x / nqb;
    qblk = blockIdx.x % nqb;
  }
  const int q0 = qblk * AQ + wave * QW;
  const bf16* qh = p.q + (size_t)head * p.n_pad * kHeadDim;
  const bf16* kh = p.k + (size_t)head * p.n_pad * kHeadDim;
  const bf16* vh = p.vt + (size_t)head * kHeadDim * p.n_pad;
  const int nkv = (p.M + AKV - 1) / AKV;

  // stream the first tiles while the queries load
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    issue_tile(kh, vh, p.n_pad, min(s, nkv - 1) * AKV, lds0 + s * STAGE_BYTES, wave, lane);

  bf16x8 qf[2][8];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qf[qb][ks] = *reinterpret_cast<const bf16x8*>(
          qh + (size_t)(q0 + qb * 32 + r32) * kHeadDim + ks * 16 + hh * 8);

  f32x16 o[4][2];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[d][qb][e] = 0.f;
  float m_ref[2] = {-INFINITY, -INFINITY}, l_sum[2] = {0.f, 0.f};
  const float sc = p.scale_log2;
  const int M = p.M;
  auto stage_ptr = [&](int tile) -> const lds_u8* { return smem + (tile % NSTAGE) * STAGE_BYTES; };
  // tile it+1 must be in LDS; past this barrier tile it-1's stage is free
  auto advance = [&](int it) {
    wait_vm<(NSTAGE - 3) * DMA_PER_TILE>();
    __syncthreads();
    issue_tile(kh, vh, p.n_pad, min(it + NSTAGE - 1, nkv - 1) * AKV,
               lds0 + ((it + NSTAGE - 1) % NSTAGE) * STAGE_BYTES, wave, lane);
  };

  wait_vm<(NSTAGE - 2) * DMA_PER_TILE>();
  __syncthreads();
  // 32-key blocks: the scores of the next block are computed before the
  // softmax of the current one, then the current block's PV.
  SHalf Sa, Sb;
  PHalf pf;
  float alpha[2];
  qk_half(Sa, smem, 0, qf, lane);
  for (int it = 0; it + 1 < nkv; ++it) {
    const lds_u8* cur = stage_ptr(it);
    const int kv0 = it * AKV;
    qk_half(Sb, cur, 1, qf, lane);
    if (softmax_half<false>(Sa, pf, m_ref, l_sum, alpha, sc, kv0, M, hh)) rescale_o(o, alpha);
    pv_half(o, cur + K_BYTES, 0, pf, lane);
    advance(it);
    qk_half(Sa, stage_ptr(it + 1), 0, qf, lane);
    if (softmax_half<false>(Sb, pf, m_ref, l_sum, alpha, sc, kv0 + 32, M, hh)) rescale_o(o, alpha);
    pv_half(o, cur + K_BYTES, 1, pf, lane);
  }
  {
    // last tile, keys past the sequence end masked
    const int it = nkv - 1;
    const lds_u8* cur = stage_ptr(it);
    const int kv0 = it * AKV;
    qk_half(Sb, cur, 1, qf, lane);
    if (softmax_half<true>(Sa, pf, m_ref, l_sum, alpha, sc, kv0, M, hh)) rescale_o(o, alpha);
    pv_half(o, cur + K_BYTES, 0, pf, lane);
    if (softmax_half<true>(Sb, pf, m_ref, l_sum, alpha, sc, kv0 + 32, M, hh)) rescale_o(o, alpha);
    pv_half(o, cur + K_BYTES, 1, pf, lane);
  }
  wait_vm<0>();

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = l_sum[qb] + xor_lane(l_sum[qb], 32);
    const float inv = 1.0f / l_tot;
    const int qi = q0 + qb * 32 + r32;
    if (qi < p.M) {
      bf16* dst = p.out + (size_t)qi * p.ldo + head * kHeadDim;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = f2bf(o[d][qb][4 * g + e] * inv);
          *reinterpret_cast<bf16x4*>(dst + d * 32 + 8 * g + 4 * hh) = v;
        }
    }
  }
}

}  // namespace

hipError_t launch_attention(const BlockShape& bs, const WsPtrs& ws,
                            hipStream_t s) {
  AttnArgs p;
  p.q = static_cast<const bf16*>(ws.q);
  p.k = static_cast<const bf16*>(ws.k);
  p.vt = static_cast<const bf16*>(ws.vt);
  p.out = static_cast<bf16*>(ws.cat);
  p.M = bs.M;
  p.n_pad = bs.n_pad;
  p.H = bs.H;
  p.ldo = bs.D + bs.F;
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)kHeadDim);
  const int nqb = (bs.M + AQ - 1) / AQ;
  hipLaunchKernelGGL(k_attention, dim3(nqb * bs.H), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace flux3
