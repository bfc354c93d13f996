// K3: full bidirectional softmax attention, flash-style, for gfx950.
//
// Every token attends to every token of the call, with no mask ("Speed,
// architecture, and how the tokens move", 15jq.com post: everything attends
// to everything in the joint stage, each stream only to itself in the
// per-mode stage -- the per-mode case is this kernel on one stream's rows).
// Queries and keys arrive RMS-normalised and rotated; the scale is
// 1/sqrt(128).
//
// Work split: a workgroup is 8 waves x 32 queries of one head, two waves per
// SIMD.  One launch attends within one sequence or within several of equal
// length (streams of the per-mode stage sharing a launch): its heads are
// then the model's heads times the sequences, each with its own first row.  A wave keeps its 32 queries in registers and computes
// S^T = K . Q^T with the 32x32x16 bf16 MFMA, so every lane owns one query
// (lane % 32) and 16 of each 32 keys; O^T = V^T . P^T then takes the
// probabilities straight from those registers as the B operand (V arrives
// transposed, keys permuted inside each group of 16 to match).
//
// Software pipeline over 64-key tiles: while the softmax of tile t runs on
// the VALU, the same wave issues the QK^T MFMAs of tile t+1 and the PV MFMAs
// of tile t-1, one of each per slot, with LDS fragments fetched four slots
// ahead; the order inside a tile is pinned with scheduling barriers.  K and
// V^T stream from global memory straight into two 4-deep LDS rings (gfx950
// direct loads, XOR-swizzled rows, spread over the tile's slots), K four
// tiles and V^T two tiles ahead of their use, one workgroup barrier per tile.
//
// Online softmax with lazy rescaling: scores are kept in the log2 domain
// (log2(e)/sqrt(128) folded into one FMA with the reference); a tile's
// probabilities are taken against a query's current reference max, and
// only when some lane's sum of them exceeds 2^TAU is the tile's own max
// taken, the reference moved and O and the running sum rescaled -- so every
// exp2(s - m) stays <= 2^TAU and fp32 / bf16 never overflow, and most tiles
// need no max at all.  Keys past the sequence end are masked in the last
// tile (the workspace pads them with zeros).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

constexpr int QW = 32;                 // queries per wave
constexpr int WAVES = 8;
constexpr int NTHREADS = 64 * WAVES;
constexpr int AQ = QW * WAVES;         // queries per workgroup
constexpr int AKV = 64;                // keys per tile
constexpr int NSTAGE = 4;              // depth of each LDS ring (tiles)
constexpr int K_ROW = kHeadDim * 2;    // 256 B: one key of K
constexpr int V_ROW = AKV * 2;         // 128 B: one dim of V^T for the tile
constexpr int K_BYTES = AKV * K_ROW;   // 16 KiB
constexpr int V_BYTES = kHeadDim * V_ROW;  // 16 KiB
constexpr int V_RING = NSTAGE * K_BYTES;   // byte offset of the V^T ring
constexpr int LDS_BYTES = NSTAGE * (K_BYTES + V_BYTES);  // 128 KiB
constexpr int DMA_PER_GROUP = 4;       // per wave: 2 for a K tile, 2 for a V^T tile
constexpr int PREFETCH = 4;            // fragment reads run this many slots ahead
constexpr float TAU = 8.0f;

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef const __attribute__((address_space(3))) bf16x8 lds_frag;

struct AttnArgs {
  const bf16 *q, *k, *vt;
  bf16* out;         // cat buffer, packed operand layout of width ldo
  float* part;       // partial-result slots of split query blocks (256 KiB each)
  int M, n_pad, H, ldo;   // H: heads of the launch, heads x sequences
  int heads;         // model heads
  // first workspace row of each sequence of M tokens the launch attends
  // within (several when equal-length streams share a launch)
  int32_t seq_row[kMaxSegs];
  float scale_log2;  // log2(e) / sqrt(head_dim)
  int groups;        // persistent workgroups G
  int dp_rounds;     // whole-unit rounds before the split tail
  int tail;          // units left to the split (0: none)
  int tail_ranges;   // ranges the tail's key tiles are cut into (<= G)
};

// A unit of work is one (head, 256-query block); unit L maps to it so that
// the units an XCD runs (L % 8 equal) share heads and keep K and V in that
// XCD's L2.
__device__ __forceinline__ void unit_coords(int L, int nqb, int H, int& head, int& qblk) {
  if (H % 8 == 0) {
    const int xcd = L & 7, idx = L >> 3;
    head = xcd * (H / 8) + idx / nqb;
    qblk = idx % nqb;
  } else {
    head = L / nqb;
    qblk = L % nqb;
  }
}

// Launch head hl -> model head and the first workspace row of its sequence.
__device__ __forceinline__ void head_rows(const AttnArgs& p, int hl, int& head, int& row0) {
  const int sq = hl / p.heads;
  head = hl - sq * p.heads;
  row0 = 0;
#pragma unroll
  for (int i = 0; i < kMaxSegs; ++i)
    if (sq == i) row0 = p.seq_row[i];
}

// Partial result of a split unit, in a 256-KiB slot: O (unnormalised, fp32)
// as float4 (wave, d, g, lane) at float4 index (16 wave + 4 d + g) 64 + lane
// -- registers o[d][4g .. 4g + 3] of that lane -- then the reference max
// m and the key sum l of query 32 wave + r at floats 32768 + (32 wave + r)
// and 33024 + (32 wave + r).
constexpr int PART_M = 32768, PART_L = 33024;

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Direct global->LDS load of 16 bytes per lane from base + voff (a uniform
// base in SGPRs, a per-lane byte offset) to LDS byte lds_off + 16 * lane.
// An asm statement (M0 set, one wait state for the M0 -> LDS-DMA hazard,
// the load) so that the compiler does not wait for it before every LDS
// read; completion is awaited explicitly with wait_vm<>.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds_off)
               : "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// LDS layouts.  K tile: key r's 256 bytes, 16-byte chunk c in slot
// c ^ (r % 16).  V^T tile: dim r's 128 bytes, chunk c in slot c ^ ((r/2) % 8).
// Both keep the 16 consecutive rows of a fragment read on distinct banks.
// A wave loads keys [8 wave, 8 wave + 8) of a K tile (2 blocks of 4 rows x
// 256 B) and dims [16 wave, 16 wave + 16) of a V^T tile (2 blocks of 8 rows
// x 128 B); the per-lane source offsets inside a tile are fixed.
struct DmaLanes {
  uint32_t k[2], v[2];   // byte offsets from the tile's first key / column
};

__device__ __forceinline__ DmaLanes dma_lanes(int n_pad, int wave, int lane) {
  DmaLanes d;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kr = 8 * wave + 4 * i + (lane >> 4);
    d.k[i] = (uint32_t)(kr * kHeadDim + ((lane & 15) ^ (kr & 15)) * 8) * 2;
    const int vr = 16 * wave + 8 * i + (lane >> 3);
    d.v[i] = (uint32_t)(vr * n_pad + ((lane & 7) ^ ((vr >> 1) & 7)) * 8) * 2;
  }
  return d;
}

__device__ __forceinline__ void issue_k(const bf16* kh, int kv0, uint32_t dst, const DmaLanes& dl,
                                        int wave) {
  const bf16* base = kh + (size_t)kv0 * kHeadDim;
#pragma unroll
  for (int i = 0; i < 2; ++i) dma16(base, dl.k[i], dst + (8 * wave + 4 * i) * K_ROW);
}
__device__ __forceinline__ void issue_v(const bf16* vh, int kv0, uint32_t dst, const DmaLanes& dl,
                                        int wave) {
  const bf16* base = vh + kv0;
#pragma unroll
  for (int i = 0; i < 2; ++i) dma16(base, dl.v[i], dst + (16 * wave + 8 * i) * V_ROW);
}

typedef f32x16 STile[2];        // S^T of one tile: [32-key block]
// P^T fragments as packed bf16 pairs: [32-key block][16-key half][pair]
typedef uint32_t PTile[2][2][4];
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 pfrag(const uint32_t (&w)[4]) {
  const u32x4 v = {w[0], w[1], w[2], w[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Keeps a value computed where it stands: earlier passes may otherwise sink
// it past the scheduling barriers into a later block.
template <class T>
__device__ __forceinline__ void pin(T& v) {
  asm volatile("" : "+v"(v));
}

// Per-query online softmax state of one lane.
struct SoftState {
  float m_ref;   // reference max, log2 domain
  float l_sum;   // running sum of exp2(s - m_ref) (fp32) over this lane's keys
  bool moved;    // wave-uniform: the last softmax region left its tile to settle()
};

constexpr float kTauExp = 256.0f;   // 2^TAU

// Score idx (key block idx / 16, register idx % 16) of this lane's query in
// a tile: keys past the sequence end are -inf under MASK.
template <bool MASK>
__device__ __forceinline__ float score(const STile& Sc, int idx, int key0, int M, int hh) {
  const int kb = idx >> 4, e = idx & 15;
  float s = Sc[kb][e];
  if constexpr (MASK) {
    const int jk = key0 + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
    s = jk < M ? s : -INFINITY;
  }
  return s;
}

// One tile's worth of pipelined work, in 32 slots.  Even slot 2j: QK^T
// MFMA j of tile t+1 (k-step j/2, key block j%2) into Sn; odd slot 2j+1: PV
// MFMA j of tile t-1 (key block j/8, 16-key half (j/4)%2, dim block j%4)
// with probabilities Pp.  Softmax of tile t (scores Sc -> Pc) rides along,
// one exponential per slot against the current reference (odd slots pack
// the pair of two slots earlier to bf16 and add it to the sum; slot 31 also
// the last pair), slot 31 checking the sum -- an even share of VALU work
// beside every MFMA.  Every exp2(s - m_ref) is
// bounded by the lane's sum
// of them, so while that sum stays within 2^TAU no probability exceeds
// 2^TAU and the tile needs no max; otherwise (or on NaN: the first tile,
// where m_ref is still -inf) `moved` is set and settle() redoes the tile
// against its true max after the region.
// A region's direct loads: none, or a callable taking the load number
// 0..3 (slots 5, 13, 21 and 29 issue one each).
struct NoLoads {
  template <class Q>
  __device__ void operator()(Q) const {}
};

template <bool QK, bool PV, bool SM, bool MASK, class Loads = NoLoads>
__device__ __forceinline__ void region(STile& Sn, uint32_t k_off, f32x16 (&o)[4], uint32_t v_off,
                                       const PTile& Pp, const STile& Sc, PTile& Pc, SoftState& st,
                                       const bf16x8 (&qf)[8], const lds_u8* smem, float scale,
                                       int key0, int M, int lane, const Loads& loads = Loads{}) {
  const int r = lane & 31, hh = lane >> 5;
  // fragment addresses: row base with the lane's swizzle term, the k-step
  // part of the chunk index is xor-ed in per slot
  const uint32_t ka = k_off + r * K_ROW + 16 * (hh ^ (r & 15));
  const uint32_t va = v_off + r * V_ROW + 16 * (hh ^ ((r >> 1) & 7));
  bf16x8 fr[32];
  auto load = [&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr ((i & 1) ? PV : QK) {
      constexpr int j = i / 2;
      uint32_t a;
      if constexpr ((i & 1) == 0)
        a = (ka ^ (32 * (j / 2))) + (j % 2) * 32 * K_ROW;
      else
        a = (va ^ (64 * (j / 8) + 32 * ((j / 4) % 2))) + (j % 4) * 32 * V_ROW;
      fr[i] = *reinterpret_cast<lds_frag*>(smem + a);
    }
  };
  static_for<0, PREFETCH>(load);

  float l = 0.f;
  f32x4 pq;   // the last four probabilities, by slot % 4
  static_for<0, 32>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    constexpr int j = i / 2;
    if constexpr ((i & 1) == 0 && QK) {
      constexpr int ks = j / 2, kb = j % 2;
      if constexpr (ks == 0)
        Sn[kb] = mfma32(fr[i], qf[0], f32x16{});
      else
        Sn[kb] = mfma32(fr[i], qf[ks], Sn[kb]);
    }
    if constexpr ((i & 1) == 1 && PV) {
      constexpr int kb = j / 8, tt = (j / 4) % 2, d = j % 4;
      o[d] = mfma32(fr[i], pfrag(Pp[kb][tt]), o[d]);
    }
    if constexpr (i + PREFETCH < 32) load(std::integral_constant<int, i + PREFETCH>{});
    if constexpr (i % 8 == 5) loads(std::integral_constant<int, i / 8>{});
    if constexpr (SM) {
      // one exponential per slot; odd slots pack the pair of two slots
      // earlier, so the conversion never waits on an exponential just issued
      pq[i & 3] = __builtin_amdgcn_exp2f(
          __builtin_fmaf(score<MASK>(Sc, i, key0, M, hh), scale, -st.m_ref));
      auto pack = [&](auto jc) {
        constexpr int idx = decltype(jc)::value;
        const f32x2 pp = {pq[idx & 3], pq[(idx + 1) & 3]};
        const bf16x2 pb = __builtin_convertvector(pp, bf16x2);
        // the running sum adds the fp32 probabilities (two full-rate adds
        // cost less than one v_dot2c of the bf16 pair)
        l += pp[0] + pp[1];
        uint32_t w = __builtin_bit_cast(uint32_t, pb);
        pin(w);
        Pc[idx >> 4][(idx >> 3) & 1][(idx & 7) >> 1] = w;
      };
      if constexpr ((i & 1) && i >= 3) pack(std::integral_constant<int, i - 3>{});
      if constexpr (i == 31) pack(std::integral_constant<int, 30>{});
      if constexpr (i == 31) {
        st.moved = __any(!(l <= kTauExp));
        st.l_sum += st.moved ? 0.f : l;
        pin(st.l_sum);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  });
}

// After a softmax region that set `moved`: the tile's max (over both lanes
// of each query) becomes the reference when it is above the current one,
// O and the running sum are rescaled by 2^(old - new), and the tile's
// probabilities and sum are taken again against it.
template <bool MASK>
__device__ __forceinline__ void settle(f32x16 (&o)[4], SoftState& st, const STile& Sc, PTile& Pc,
                                       float scale, int key0, int M, int lane) {
  if (!st.moved) return;
  const int hh = lane >> 5;
  float m = -INFINITY;
#pragma unroll
  for (int idx = 0; idx < 32; ++idx) m = fmaxf(m, score<MASK>(Sc, idx, key0, M, hh));
  m *= scale;
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                   false, false);
  const float m_new = fmaxf(st.m_ref, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
  const float alpha = __builtin_amdgcn_exp2f(st.m_ref - m_new);
  st.m_ref = m_new;
  float l = 0.f;
#pragma unroll
  for (int idx = 0; idx < 32; idx += 2) {
    f32x2 pp;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      pp[u] = __builtin_amdgcn_exp2f(
          __builtin_fmaf(score<MASK>(Sc, idx + u, key0, M, hh), scale, -m_new));
    const bf16x2 pb = __builtin_convertvector(pp, bf16x2);
    l += pp[0] + pp[1];
    Pc[idx >> 4][(idx >> 3) & 1][(idx & 7) >> 1] = __builtin_bit_cast(uint32_t, pb);
  }
  st.l_sum = st.l_sum * alpha + l;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
}

// Attention of one unit (head, query block qblk) over key tiles
// [t0, t0 + nt): normalised into the concatenation buffer when slot is
// null, else the unnormalised O with its m and l into the slot.
__device__ __forceinline__ void attend(const AttnArgs& p, const lds_u8* smem, uint32_t lds0,
                                       int hl, int qblk, int t0, int nt, float* slot) {
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int r32 = lane & 31, hh = lane >> 5;
  const int q0 = qblk * AQ + wave * QW;
  int head, row0;
  head_rows(p, hl, head, row0);
  const bf16* qh = p.q + ((size_t)head * p.n_pad + row0) * kHeadDim;
  const bf16* kh = p.k + ((size_t)head * p.n_pad + row0) * kHeadDim;
  const bf16* vh = p.vt + (size_t)head * kHeadDim * p.n_pad + row0;
  const int M = p.M;
  const float sc = p.scale_log2;
  const int kbase = t0 * AKV;   // first key of the range

  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(qh + (size_t)(q0 + r32) * kHeadDim + ks * 16 + hh * 8);

  // DMA group g (issued at the top of tile g of the range, or over tile g's
  // slots in the steady loop): K tile g+4 and V^T tile g+2, indices clamped
  // to the range; the prologue issues groups -4..-1.
  const DmaLanes dl = dma_lanes(p.n_pad, wave, lane);
  auto k_stage = [](int tile) { return (uint32_t)((tile & (NSTAGE - 1)) * K_BYTES); };
  auto v_stage = [](int tile) { return (uint32_t)(V_RING + (tile & (NSTAGE - 1)) * V_BYTES); };
  auto issue_group = [&](int g) {
    const int kt = g + 4, vt = g + 2;
    issue_k(kh, kbase + min(kt, nt - 1) * AKV, lds0 + k_stage(kt), dl, wave);
    issue_v(vh, kbase + max(0, min(vt, nt - 1)) * AKV, lds0 + v_stage(vt), dl, wave);
  };
#pragma unroll
  for (int g = -4; g < 0; ++g) issue_group(g);

  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  SoftState st{-INFINITY, 0.f, false};
  STile S0, S1;
  PTile P0, P1;

  // top of tile it: K tile it+1 and V^T tile it-1 (group it-3) resident in
  // every wave's part; past the barrier K tile it and V^T tile it-2 are no
  // longer read, and group it refills those stages
  auto top = [&](int it) {
    wait_vm<2 * DMA_PER_GROUP>();
    __syncthreads();
    issue_group(it);
  };
  // In the steady loop a tile's group goes out one load per eight slots of
  // its region instead of all four at the top: eight waves issuing 32 loads
  // at once after the barrier fill the vector memory queue, and a wave
  // stalled behind a queued load stalls its MFMAs too.
  auto top_wait = [&]() {
    wait_vm<2 * DMA_PER_GROUP>();
    __syncthreads();
  };
  auto spread_group = [&](int g) {
    return [&, g](auto qc) {
      constexpr int q = decltype(qc)::value;   // K halves, then V^T halves
      if constexpr (q < 2) {
        const int kt = g + 4;
        const bf16* base = kh + (size_t)(kbase + min(kt, nt - 1) * AKV) * kHeadDim;
        dma16(base, dl.k[q], lds0 + k_stage(kt) + (8 * wave + 4 * q) * K_ROW);
      } else {
        const int vt = g + 2;
        const bf16* base = vh + kbase + max(0, min(vt, nt - 1)) * AKV;
        dma16(base, dl.v[q - 2], lds0 + v_stage(vt) + (16 * wave + 8 * (q - 2)) * V_ROW);
      }
    };
  };

  // scores of tile 0 (group -4 landed: the later 3 groups may be in flight)
  wait_vm<3 * DMA_PER_GROUP>();
  __syncthreads();
  region<true, false, false, false>(S0, k_stage(0), o, 0, P1, S1, P1, st, qf, smem, sc, 0, M, lane);

  // the range's last tile runs with the key mask (a no-op unless it is the
  // sequence's last tile)
  top(0);
  if (nt == 1) {
    region<false, false, true, true>(S1, 0, o, 0, P1, S0, P0, st, qf, smem, sc, kbase, M, lane);
    settle<true>(o, st, S0, P0, sc, kbase, M, lane);
    wait_vm<0>();
    __syncthreads();
    region<false, true, false, false>(S1, 0, o, v_stage(0), P0, S0, P1, st, qf, smem, sc, 0, M, lane);
  } else {
    region<true, false, true, false>(S1, k_stage(1), o, 0, P1, S0, P0, st, qf, smem, sc, kbase, M,
                                     lane);
    settle<false>(o, st, S0, P0, sc, kbase, M, lane);
    int it = 1;
    for (; it + 1 < nt - 1; it += 2) {
      // it odd: scores in S1, probabilities to P1; then it+1 even
      top_wait();
      region<true, true, true, false>(S0, k_stage(it + 1), o, v_stage(it - 1), P0, S1, P1, st, qf,
                                      smem, sc, kbase + it * AKV, M, lane, spread_group(it));
      settle<false>(o, st, S1, P1, sc, kbase + it * AKV, M, lane);
      top_wait();
      region<true, true, true, false>(S1, k_stage(it + 2), o, v_stage(it), P1, S0, P0, st, qf,
                                      smem, sc, kbase + (it + 1) * AKV, M, lane, spread_group(it + 1));
      settle<false>(o, st, S0, P0, sc, kbase + (it + 1) * AKV, M, lane);
    }
    if (it < nt - 1) {
      // it = nt-2 (odd), then the last tile nt-1 (even)
      top(it);
      region<true, true, true, false>(S0, k_stage(it + 1), o, v_stage(it - 1), P0, S1, P1, st, qf,
                                      smem, sc, kbase + it * AKV, M, lane);
      settle<false>(o, st, S1, P1, sc, kbase + it * AKV, M, lane);
      top(it + 1);
      region<false, true, true, true>(S1, 0, o, v_stage(it), P1, S0, P0, st, qf, smem, sc,
                                      kbase + (it + 1) * AKV, M, lane);
      settle<true>(o, st, S0, P0, sc, kbase + (it + 1) * AKV, M, lane);
      wait_vm<0>();
      __syncthreads();
      region<false, true, false, false>(S1, 0, o, v_stage(it + 1), P0, S0, P1, st, qf, smem, sc, 0,
                                        M, lane);
    } else {
      // it = nt-1 (odd) is the last tile
      top(it);
      region<false, true, true, true>(S0, 0, o, v_stage(it - 1), P0, S1, P1, st, qf, smem, sc,
                                      kbase + it * AKV, M, lane);
      settle<true>(o, st, S1, P1, sc, kbase + it * AKV, M, lane);
      wait_vm<0>();
      __syncthreads();
      region<false, true, false, false>(S0, 0, o, v_stage(it), P1, S1, P0, st, qf, smem, sc, 0, M,
                                        lane);
    }
  }

  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.l_sum),
                                                   __float_as_uint(st.l_sum), false, false);
  const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  if (slot) {
    float4* so = reinterpret_cast<float4*>(slot) + (size_t)wave * 16 * 64 + lane;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        so[(4 * d + g) * 64] = make_float4(o[d][4 * g], o[d][4 * g + 1], o[d][4 * g + 2],
                                           o[d][4 * g + 3]);
    if (hh == 0) {
      slot[PART_M + wave * 32 + r32] = st.m_ref;
      slot[PART_L + wave * 32 + r32] = l_tot;
    }
    return;
  }
  const float inv = 1.0f / l_tot;
  const int qi = q0 + r32;
  if (qi < M) {
    // the concatenation buffer is in the packed operand layout
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = f2bf(o[d][4 * g + e] * inv);
        const int col = head * kHeadDim + d * 32 + 8 * g + 4 * hh;
        *reinterpret_cast<bf16x4*>(p.out + packed_index(row0 + qi, col, p.ldo)) = v;
      }
  }
}

// Persistent workgroups: dp_rounds rounds of whole units (G at a time),
// then, if the leftover units would leave most of a round idle, their key
// tiles split evenly over tail_ranges ranges (SplitK: one unit = its nkv key
// tiles).  A unit a range covers whole is finished at once; the partial
// results of a unit cut by range boundaries go to slots that
// k_attention_fixup merges.
__global__ __launch_bounds__(NTHREADS, 1) void k_attention(AttnArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[LDS_BYTES];
  const lds_u8* smem = (const lds_u8*)smem_raw;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem_raw;
  const int nqb = (p.M + AQ - 1) / AQ;
  const int nkv = (p.M + AKV - 1) / AKV;
  const int units = nqb * p.H;
  const int G = p.groups;
  // the tail range of this workgroup (empty without a tail)
  SplitK sk;
  sk.nk = nkv;
  sk.G = p.tail_ranges > 0 ? p.tail_ranges : 1;
  sk.total = (int64_t)p.tail * nkv;
  const int v = range_of_block(blockIdx.x, G);
  int64_t s = 0, s_end = 0;
  if (p.tail > 0 && v < sk.G) {
    s = sk.start(v);
    s_end = sk.start(v + 1);
  }
  const int unit0 = p.dp_rounds * G;
  // one loop over this workgroup's work items -- whole units, then tail
  // segments -- so that the unit body is instantiated once
  int r = 0;
  bool first = true;
  for (;;) {
    int head, qblk, t0, nt;
    float* slot = nullptr;
    if (r < p.dp_rounds && r * G + (int)blockIdx.x < units) {
      unit_coords(r * G + blockIdx.x, nqb, p.H, head, qblk);
      t0 = 0;
      nt = nkv;
      ++r;
    } else if (s < s_end) {
      r = p.dp_rounds;
      const int u = (int)(s / nkv);
      const int kb = (int)(s - (int64_t)u * nkv);
      const int ke = (int)min<int64_t>(nkv, kb + (s_end - s));
      unit_coords(unit0 + u, nqb, p.H, head, qblk);
      t0 = kb;
      nt = ke - kb;
      if (nt != nkv) slot = p.part + (size_t)sk.slot(v, u) * 65536;
      s += nt;
    } else {
      break;
    }
    if (!first) __syncthreads();   // the previous item's LDS reads are done
    first = false;
    attend(p, smem, lds0, head, qblk, t0, nt, slot);
  }
}

// Merges the partial results of every tail unit cut by a range boundary:
// m = max m_i, O = sum 2^(m_i - m) O_i, l = sum 2^(m_i - m) l_i, out = O / l.
// Workgroup (i, w) looks at the boundary between ranges i and i + 1, takes
// its unit if no earlier boundary falls inside it, and merges the 32
// queries of attention wave w.  Its NW waves share the unit's pieces (wave
// k takes pieces k, k + NW, ..., two at a time, folding them into a running
// (m, l, O) the way the attention loop does); waves 1 .. NW-1 hand their
// running results to wave 0 through LDS, and wave 0 folds them in, in wave
// order, and writes the output.  A lane handles the registers one attention
// lane held.  One wave serves units of a few pieces; four share the many
// pieces of a unit cut into short ranges.

__device__ __forceinline__ void fold_piece(float& m, float& l, float4 (&acc)[16], float mv, float lv,
                                           const float4 (&o)[16]) {
  const float mn = fmaxf(m, mv);
  const float a = __builtin_amdgcn_exp2f(m - mn), b = __builtin_amdgcn_exp2f(mv - mn);
  l = a * l + b * lv;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    acc[j].x = a * acc[j].x + b * o[j].x;
    acc[j].y = a * acc[j].y + b * o[j].y;
    acc[j].z = a * acc[j].z + b * o[j].z;
    acc[j].w = a * acc[j].w + b * o[j].w;
  }
  m = mn;
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void k_attention_fixup(AttnArgs p) {
  constexpr int NX = NW > 1 ? NW - 1 : 1;   // LDS hand-over slots
  __shared__ float4 s_acc[NX][16][64];
  __shared__ float s_m[NX][64], s_l[NX][64];
  const int nqb = (p.M + AQ - 1) / AQ;
  const int nkv = (p.M + AKV - 1) / AKV;
  SplitK sk;
  sk.nk = nkv;
  sk.G = p.tail_ranges;
  sk.total = (int64_t)p.tail * nkv;
  const int i = blockIdx.x / WAVES, wave = blockIdx.x % WAVES;
  const int64_t b = sk.start(i + 1);
  if (b % nkv == 0) return;                        // boundary on a unit edge
  const int u = (int)(b / nkv);
  if (sk.start(i) > (int64_t)u * nkv) return;      // an earlier boundary owns the unit
  const int v_first = sk.range_of((int64_t)u * nkv);
  const int v_last = sk.range_of((int64_t)(u + 1) * nkv - 1);
  const int k = threadIdx.x >> 6, lane = threadIdx.x & 63, r32 = lane & 31, hh = lane >> 5;
  const int qw = wave * 32 + r32;                  // query within the unit

  // this wave's running merge of pieces v_first + k, + NW, ...  A range of
  // at least one key tile always holds a live key, so every stored m is
  // finite; an empty range (start(v + 1) == start(v)) stored nothing.
  float m = -INFINITY, l = 0.f;
  float4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int v0 = v_first + k; v0 <= v_last; v0 += 2 * NW) {
    const int v1 = v0 + NW;
    const bool has0 = sk.start(v0 + 1) != sk.start(v0);
    const bool has1 = v1 <= v_last && sk.start(v1 + 1) != sk.start(v1);
    const float* s0 = p.part + (size_t)sk.slot(has0 ? v0 : v_first, u) * 65536;
    const float* s1 = p.part + (size_t)sk.slot(has1 ? v1 : v_first, u) * 65536;
    float4 o0[16], o1[16];
    const float4* so0 = reinterpret_cast<const float4*>(s0) + (size_t)wave * 16 * 64 + lane;
    const float4* so1 = reinterpret_cast<const float4*>(s1) + (size_t)wave * 16 * 64 + lane;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      o0[j] = so0[j * 64];
      o1[j] = so1[j * 64];
    }
    const float m0 = s0[PART_M + qw], l0 = s0[PART_L + qw];
    const float m1 = s1[PART_M + qw], l1 = s1[PART_L + qw];
    if (has0) fold_piece(m, l, acc, m0, l0, o0);
    if (has1) fold_piece(m, l, acc, m1, l1, o1);
  }
  if (NW > 1) {
    if (k > 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s_acc[k - 1][j][lane] = acc[j];
      s_m[k - 1][lane] = m;
      s_l[k - 1][lane] = l;
    }
    __syncthreads();
    if (k > 0) return;
    // wave 0 folds in the other waves' results, in wave order
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) {
      const float mw = s_m[w][lane];
      if (mw == -INFINITY) continue;   // a wave that found no piece
      float4 ow[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) ow[j] = s_acc[w][j][lane];
      fold_piece(m, l, acc, mw, s_l[w][lane], ow);
    }
  }
  int hl, qblk, head, row0;
  unit_coords(p.dp_rounds * p.groups + u, nqb, p.H, hl, qblk);
  head_rows(p, hl, head, row0);
  const int qi = qblk * AQ + qw;
  if (qi >= p.M) return;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 x = acc[4 * d + g];
      bf16x4 o;
      o[0] = f2bf(x.x * inv);
      o[1] = f2bf(x.y * inv);
      o[2] = f2bf(x.z * inv);
      o[3] = f2bf(x.w * inv);
      const int col = head * kHeadDim + d * 32 + 8 * g + 4 * hh;
      *reinterpret_cast<bf16x4*>(p.out + packed_index(row0 + qi, col, p.ldo)) = o;
    }
}

}  // namespace

hipError_t launch_attention(const BlockShape& bs, const WsPtrs& ws, const int32_t* seq_row,
                            int n_seq, hipStream_t s) {
  if (n_seq < 1 || n_seq > kMaxSegs) return hipErrorInvalidValue;
  AttnArgs p;
  p.q = static_cast<const bf16*>(ws.q);
  p.k = static_cast<const bf16*>(ws.k);
  p.vt = static_cast<const bf16*>(ws.vt);
  p.out = static_cast<bf16*>(ws.cat);
  p.part = static_cast<float*>(ws.part);
  p.M = bs.M;
  p.n_pad = bs.n_pad;
  p.heads = bs.H;
  p.H = bs.H * n_seq;
  for (int i = 0; i < kMaxSegs; ++i) p.seq_row[i] = i < n_seq ? seq_row[i] : 0;
  p.ldo = bs.D + bs.F;
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)kHeadDim);
  const int nqb = (bs.M + AQ - 1) / AQ;
  const int nkv = (bs.M + AKV - 1) / AKV;
  const int units = nqb * p.H;
  const int G = stream_k_groups();
  p.groups = G;
  p.dp_rounds = units / G;
  p.tail = units % G;
  // a tail filling most of a round runs whole (as does every tail without a
  // partial-slot region, ws.part null); a thin one has its key tiles spread
  // over up to G ranges of at least 4 tiles each
  if (p.tail * 10 > G * 7 || ws.part == nullptr) {
    p.dp_rounds += 1;
    p.tail = 0;
  }
  p.tail_ranges = 0;
  if (p.tail > 0) {
    const int64_t items = (int64_t)p.tail * nkv;
    p.tail_ranges = (int)std::min<int64_t>(G, std::max<int64_t>(1, items / 4));
  }
  hipLaunchKernelGGL(k_attention, dim3(G), dim3(NTHREADS), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.tail_ranges < 2) return e;
  // pieces a unit can be cut into: ranges hold at least items / ranges tiles
  const int64_t per_range = (int64_t)p.tail * nkv / p.tail_ranges;
  const int64_t pieces = (nkv + per_range - 1) / per_range + 1;
  if (pieces <= 4)
    hipLaunchKernelGGL(k_attention_fixup<1>, dim3((p.tail_ranges - 1) * WAVES), dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(k_attention_fixup<4>, dim3((p.tail_ranges - 1) * WAVES), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace flux3
