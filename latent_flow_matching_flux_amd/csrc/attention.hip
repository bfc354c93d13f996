// K3: full bidirectional softmax attention, flash-style, for gfx950.
//
// Every token attends to every token of the call, with no mask ("Speed,
// architecture, and how the tokens move", 15jq.com post: everything attends
// to everything in the joint stage, each stream only to itself in the
// per-mode stage -- the per-mode case is this kernel on one stream's rows).
// Queries and keys arrive RMS-normalised and rotated; the scale is
// 1/sqrt(128).
//
// Work split: one workgroup = 4 waves x 32 queries of one head.  Each wave
// keeps its queries in registers and computes S^T = K . Q^T with the
// 32x32x16 bf16 MFMA, so that every lane owns one query (lane % 32) and 16
// of each 32 keys.  The online softmax (running max and sum, exp2 with
// log2(e)/sqrt(128) folded into the scale) is per lane plus one exchange
// with lane ^ 32.  O^T = V^T . P^T reuses the probabilities straight from
// the accumulator registers as the B operand; V arrives transposed with keys
// permuted inside each group of 16 to match.  K and V^T tiles of 64 keys are
// staged through LDS, double-buffered.  Keys past the sequence end are
// masked to -inf (the workspace pads them with zeros).
#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

constexpr int AQ = 128;          // queries per workgroup
constexpr int AKV = 64;          // keys per tile
constexpr int KLD = 128 + 8;     // K tile row stride (elements)
constexpr int VLD = AKV + 8;     // V^T tile row stride (elements)
constexpr int K_ELEMS = AKV * KLD;
constexpr int V_ELEMS = kHeadDim * VLD;

struct AttnArgs {
  const bf16 *q, *k, *vt;
  bf16* out;         // cat buffer, row stride ldo
  int M, n_pad, H, ldo;
  float scale_log2;  // log2(e) / sqrt(head_dim)
};

__device__ __forceinline__ void load_kv(u32x4 (&rk)[4], u32x4 (&rv)[4],
                                        const bf16* kh, const bf16* vh,
                                        int n_pad, int kv0, int t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = t + 256 * i;
    rk[i] = *reinterpret_cast<const u32x4*>(kh + (size_t)(kv0 + (id >> 4)) * kHeadDim + (id & 15) * 8);
    rv[i] = *reinterpret_cast<const u32x4*>(vh + (size_t)(id >> 3) * n_pad + kv0 + (id & 7) * 8);
  }
}

__device__ __forceinline__ void store_kv(bf16* Ks, bf16* Vs, const u32x4 (&rk)[4],
                                         const u32x4 (&rv)[4], int t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = t + 256 * i;
    *reinterpret_cast<u32x4*>(Ks + (id >> 4) * KLD + (id & 15) * 8) = rk[i];
    *reinterpret_cast<u32x4*>(Vs + (id >> 3) * VLD + (id & 7) * 8) = rv[i];
  }
}

__global__ __launch_bounds__(256, 2) void k_attention(AttnArgs p) {
  __shared__ bf16 Ks[2][K_ELEMS];
  __shared__ bf16 Vs[2][V_ELEMS];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int r32 = lane & 31, hi = lane >> 5;
  const int head = blockIdx.y;
  const int q0 = blockIdx.x * AQ;
  const bf16* qh = p.q + (size_t)head * p.n_pad * kHeadDim;
  const bf16* kh = p.k + (size_t)head * p.n_pad * kHeadDim;
  const bf16* vh = p.vt + (size_t)head * kHeadDim * p.n_pad;

  const int qi = q0 + wave * 32 + r32;
  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(qh + (size_t)qi * kHeadDim + ks * 16 + hi * 8);

  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nkv = (p.M + AKV - 1) / AKV;
  u32x4 rk[4], rv[4];
  load_kv(rk, rv, kh, vh, p.n_pad, 0, t);
  store_kv(Ks[0], Vs[0], rk, rv, t);
  __syncthreads();

  for (int it = 0; it < nkv; ++it) {
    const int cur = it & 1;
    if (it + 1 < nkv) load_kv(rk, rv, kh, vh, p.n_pad, (it + 1) * AKV, t);

    // S^T for 64 keys x this wave's 32 queries
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &Ks[cur][(kb * 32 + r32) * KLD + ks * 16 + hi * 8]);
        s[kb] = mfma32(a, qf[ks], s[kb]);
      }
    }
    // scale, mask, running max
    const int kv0 = it * AKV;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = kv0 + kb * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
        const float v = j < p.M ? s[kb][e] * p.scale_log2 : -INFINITY;
        s[kb][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, xor_lane(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = exp2f(s[kb][e] - m_new);
        l_run += pv;
        pf[kb][e >> 3][e & 7] = f2bf(pv);
      }
    // O^T += V^T . P^T
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              &Vs[cur][(d * 32 + r32) * VLD + kb * 32 + tt * 16 + hi * 8]);
          o[d] = mfma32(a, pf[kb][tt], o[d]);
        }
    if (it + 1 < nkv) store_kv(Ks[cur ^ 1], Vs[cur ^ 1], rk, rv, t);
    __syncthreads();
  }

  const float l_tot = l_run + xor_lane(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (qi < p.M) {
    bf16* dst = p.out + (size_t)qi * p.ldo + head * kHeadDim;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = f2bf(o[d][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(dst + d * 32 + 8 * g + 4 * hi) = v;
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
  dim3 grid((bs.M + AQ - 1) / AQ, bs.H);
  hipLaunchKernelGGL(k_attention, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace flux3
