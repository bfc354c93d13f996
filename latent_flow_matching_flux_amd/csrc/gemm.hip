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
// A rowwise-FP8 variant of both (the rowwise-FP8 single file of the
// release post, section on smaller GPUs and single files) reads e4m3 codes
// of h / [o | act] (one scale per token row) and of the weights (one scale
// per output row) through the same pipeline: a 128-byte LDS slice row then
// holds 128 codes, consumed by two 32x32x64 fp8 MFMA steps, and the row
// scales multiply each finished product tile.
//
// Both operands are K-contiguous ("NT"): C[m][n] = sum_k A[m][k] * B[n][k],
// with B in torch Linear layout [out][in].  Tile 256 x 256 x 64, 4 waves in
// a 2 x 2 arrangement, each wave 128 x 128 = 4 x 4 blocks of the 32x32x16
// bf16 MFMA, fp32 accumulators.  A and B k-slices stream from global memory
// straight into LDS (gfx950 global_load_lds_dwordx4, no staging registers),
// XOR-swizzled instead of padded, through a ring of LDS buffers that keeps
// several slices in flight (one barrier per slice); fragment reads and the
// loads are interleaved with the MFMAs.  Workgroups are remapped so that the workgroups resident on one
// XCD (every 8th id) cover a compact group of C tiles and share A and B
// slices in that XCD's L2.
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace flux3 {

namespace {

constexpr int BM = 256, BN = 256;
constexpr int NTHREADS = 256;
constexpr int GROUP_M = 8;

constexpr int BK = 64;                   // k depth of one LDS slice

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gvoid;

// Geometry of one operand's k-slice in LDS.  Tile row r (256 rows per
// operand) occupies ROW_BYTES contiguous bytes, no padding; its 16-byte
// chunk c sits in slot c ^ ((r / SWZ_DIV) % CPR), where SWZ_DIV rows span
// one 256-byte bank cycle.  With 64 banks this keeps the MFMA fragment
// reads (32 consecutive rows, one chunk, per half-wave) conflict-free, and
// lets each wave fill whole 1-KiB blocks with direct global->LDS loads:
// lane l of a block writes slot l % CPR of row l / CPR, so it fetches chunk
// (l % CPR) ^ swizzle(row).
constexpr int ROW_BYTES = BK * 2;
constexpr int CPR = ROW_BYTES / 16;
constexpr int ROWS_PER_KB = 1024 / ROW_BYTES;
constexpr int SWZ_DIV = 256 / ROW_BYTES;
constexpr int OP_BYTES = BM * ROW_BYTES;               // one operand's slice: 32 KiB
// Each operand has its own ring of slices.  The one streaming the weights
// (row-major, 8 rows per load, often from beyond L2) keeps 3 buffers, so its
// loads run two slices ahead; the packed activation keeps 2 (one ahead).
constexpr int DEEP_STAGES = 3, SHALLOW_STAGES = 2;
constexpr int LDS_BYTES = (DEEP_STAGES + SHALLOW_STAGES) * OP_BYTES;
constexpr int LOADS_PER_OP = 64 / ROWS_PER_KB;         // 1-KiB blocks per wave per operand slice
// MFMA k-steps per slice: a slice row holds 128 bytes, 64 bf16 values (four
// 16-deep bf16 steps) or 128 fp8 codes (two 64-deep fp8 steps).
template <bool F8>
constexpr int KSTEPS = F8 ? 2 : 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS rings too large");
static_assert(BK == 64 && SWZ_DIV == 2 && CPR == 8,
              "the packed operand layout holds 64-wide k blocks with this swizzle");
static_assert(LOADS_PER_OP == 8 && KSTEPS<false> == 4 && KSTEPS<true> == 2,
              "load schedule: 8 loads per operand and slice");

struct Acc {
  f32x16 c[4][4];
};

// Tile coordinates of linear tile index lin: GROUP_M M-tiles at a time,
// M fastest within a group.  tile_coords below gives workgroup id b its
// tile: XCD-major (ids b, b+8, ... share an XCD and take consecutive linear
// indices of one region of total / 8), so one XCD's tiles are neighbours.
__device__ __forceinline__ void lin_coords(int lin, int n_m, int n_n, int& mt, int& nt) {
  const int group = GROUP_M * n_n;
  const int g = lin / group;
  const int first_m = g * GROUP_M;
  const int gm = min(n_m - first_m, GROUP_M);
  const int in = lin - g * group;
  mt = first_m + in % gm;
  nt = in / gm;
}

__device__ __forceinline__ void tile_coords(int b, int n_m, int n_n, int& mt,
                                            int& nt) {
  const int total = n_m * n_n;
  const int per = total / 8;
  lin_coords((b < per * 8) ? (b % 8) * per + b / 8 : b, n_m, n_n, mt, nt);
}

// Linear index of the t-th tile left after workgroup ids [0, tile0) took
// theirs through tile_coords: those ids fill, in region x = [x per, (x + 1)
// per), its first ceil((min(tile0, 8 per) - x) / 8) indices and, past the
// regions, every index below tile0; the rest is taken region by region, in
// increasing order.
__device__ __forceinline__ int tail_lin(int t, int total, int tile0) {
  const int per = total / 8;
  const int m8 = min(tile0, 8 * per);
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const int done = (m8 - x + 7) / 8;
    if (t < per - done) return x * per + done + t;
    t -= per - done;
  }
  return max(8 * per, tile0) + t;
}

// Where this wave's share of one operand tile comes from: wave w loads tile
// rows [64w, 64w + 64).  Row-major operand: the 32-row runs 2w (lo) and
// 2w + 1 (hi) each have a wave-uniform base pointer (first row, k = 0) and
// all rows share the stride ld.  Packed operand: lo is the first of the 8
// 8-row blocks at k = 0 (row 64w's row-major offset, row * K), ld the
// stride between 8-row blocks (8 K); hi is unused.
struct Src {
  const bf16* lo;
  const bf16* hi;
  int ld;
};

// One direct global->LDS load of 16 bytes per lane: lane l's data lands at
// LDS byte lds_off + 16 l.  Written as a two-instruction asm statement (M0
// set, one wait state for the M0 -> LDS-DMA hazard, then the load) so that
// the compiler does not track it: it would otherwise wait for every such
// load in flight before any LDS read, collapsing the multi-slice pipeline.
// The statement has no register outputs; the address is consumed at issue.
// Completion is awaited explicitly with wait_vm<>.
__device__ __forceinline__ void dma16(const bf16* g, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_off)
               : "m0");
}

// The same load from base + voff: a base uniform over the wave (SGPRs) and
// a per-lane byte offset, so that a slice's k offset moves only the scalar
// base and the lanes' offsets stay fixed over the main loop.
__device__ __forceinline__ void dma16s(const bf16* base, uint32_t voff, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds_off)
               : "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// The i-th of this wave's direct loads for one slice (A blocks first, then
// B): LOADS_PER_OP 1-KiB blocks per operand, rows [64w, 64w + 64) of the tile.
// A row-major operand (P false) fetches each lane's chunk from its row with
// the LDS swizzle applied; a packed one (P true) already holds 1-KiB blocks
// in LDS order, so lane l fetches bytes [16 l, 16 l + 16) of its block.
// koff is the slice's k offset in elements of the operand's layout.
template <int I, bool P>
__device__ __forceinline__ void issue_load(const Src& S, int koff, uint32_t dst, int wave,
                                           int lane) {
  constexpr int i = I % LOADS_PER_OP;
  const bf16* base;
  uint32_t off;   // bytes from the slice's base; fits 32 bits for rows shorter than 2^24 elements
  if constexpr (P) {
    base = S.lo + koff;
    off = (uint32_t)(i * S.ld + lane * 8) * 2u;
  } else {
    const int rsub = lane / CPR, slot = lane % CPR;
    const int rr = i * ROWS_PER_KB + rsub;                 // row within this wave's 64
    const int c = slot ^ ((rr / SWZ_DIV) % CPR);
    base = (i * ROWS_PER_KB < 32 ? S.lo : S.hi) + koff;
    off = (uint32_t)((rr & 31) * S.ld + c * 8) * 2u;
  }
  dma16s(base, off, dst + (uint32_t)((64 * wave + i * ROWS_PER_KB) * ROW_BYTES));
}

// Element offset of k (a multiple of BK) in a row-major or packed operand.
template <bool P>
__device__ __forceinline__ int k_offset(int k) {
  return P ? k * 8 : k;
}

// One k-step's operand fragments of a wave: 4 A and 4 B blocks of 32 rows.
template <bool F8>
struct Frags {
  bf16x8 a[4], b[4];
};
template <>
struct Frags<true> {
  i32x8 a[4], b[4];
};

// The fragment reads of k-step kk for block Q (Q < 4: A block Q, else B
// block Q - 4).  bf16: one 16-byte chunk per lane (lane half h takes chunk
// 2 kk + h).  fp8: two chunks per lane, 32 consecutive codes (lane half h
// takes chunks 4 kk + 2 h and 4 kk + 2 h + 1).
template <int Q, bool F8>
__device__ __forceinline__ void read_frag(Frags<F8>& f, const lds_u8* As, const lds_u8* Bs,
                                          int wm, int wn, int lane, int kk) {
  const int r = lane & 31;
  const int swz = (r / SWZ_DIV) % CPR;
  const lds_u8* row = Q < 4 ? As + (wm * 128 + Q * 32 + r) * ROW_BYTES
                            : Bs + (wn * 128 + (Q - 4) * 32 + r) * ROW_BYTES;
  if constexpr (!F8) {
    typedef const __attribute__((address_space(3))) bf16x8 lds_frag;
    const bf16x8 v = *reinterpret_cast<lds_frag*>(row + (((2 * kk + (lane >> 5)) ^ swz) << 4));
    if constexpr (Q < 4) f.a[Q] = v; else f.b[Q - 4] = v;
  } else {
    typedef const __attribute__((address_space(3))) u32x4 lds_chunk;
    const int c0 = 4 * kk + 2 * (lane >> 5);
    const u32x4 lo = *reinterpret_cast<lds_chunk*>(row + ((c0 ^ swz) << 4));
    const u32x4 hi = *reinterpret_cast<lds_chunk*>(row + (((c0 + 1) ^ swz) << 4));
    const i32x8 v = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    if constexpr (Q < 4) f.a[Q] = v; else f.b[Q - 4] = v;
  }
}

// Per-workgroup stream state.
// Everything is held by value (wave-uniform values in scalar registers): a
// pointer to a stack copy would be spilled and re-read from scratch, and
// that read's wait would also wait for every direct load in flight.
// DEEP_B: B is the weight operand (3-slice ring), A the activation (2);
// otherwise the other way round.
template <bool PA, bool PB, bool DEEP_B>
struct Stream {
  static constexpr int SA = DEEP_B ? SHALLOW_STAGES : DEEP_STAGES;
  static constexpr int SB = DEEP_B ? DEEP_STAGES : SHALLOW_STAGES;
  static constexpr int B_BASE = SA * OP_BYTES;
  lds_u8* smem;
  uint32_t lds0;       // LDS byte address of smem
  Src A, B0, B1;
  int nk0;             // slices [0, nk0) take B rows from B0, later ones from B1
  int k_begin, nk;     // this call covers slices [k_begin, k_begin + nk)
  int wave, lane, wm, wn;
  // the next A and B slices to load, spread over the current slice's MFMAs
  int ld_k_a;
  uint32_t ld_dst_a;
  Src ld_b;            // B source of that slice, offset to its k
  uint32_t ld_dst_b;

  // s counts slices from k_begin; past the end the last slice is re-fetched
  // into a free buffer
  __device__ __forceinline__ void set_load_a(int s) {
    ld_dst_a = lds0 + (uint32_t)((s % SA) * OP_BYTES);
    s = k_begin + min(s, nk - 1);
    ld_k_a = k_offset<PA>(s * BK);
  }
  __device__ __forceinline__ void set_load_b(int s) {
    ld_dst_b = lds0 + (uint32_t)(B_BASE + (s % SB) * OP_BYTES);
    s = k_begin + min(s, nk - 1);
    const bool ph0 = s < nk0;
    const int kb = k_offset<PB>(ph0 ? s * BK : (s - nk0) * BK);
    ld_b.lo = (ph0 ? B0.lo : B1.lo) + kb;
    ld_b.hi = (ph0 ? B0.hi : B1.hi) + kb;
    ld_b.ld = ph0 ? B0.ld : B1.ld;
  }
  __device__ __forceinline__ void set_load_shallow(int s) {
    if constexpr (DEEP_B) set_load_a(s); else set_load_b(s);
  }
  __device__ __forceinline__ void set_load_deep(int s) {
    if constexpr (DEEP_B) set_load_b(s); else set_load_a(s);
  }
  // load I of the shallow (first) or deep (second) operand's pending slice
  template <int I>
  __device__ __forceinline__ void load_shallow() const {
    if constexpr (DEEP_B)
      issue_load<I, PA>(A, ld_k_a, ld_dst_a, wave, lane);
    else
      issue_load<I, PB>(ld_b, 0, ld_dst_b, wave, lane);
  }
  template <int I>
  __device__ __forceinline__ void load_deep() const {
    if constexpr (DEEP_B)
      issue_load<I, PB>(ld_b, 0, ld_dst_b, wave, lane);
    else
      issue_load<I, PA>(A, ld_k_a, ld_dst_a, wave, lane);
  }
  template <int... I>
  __device__ __forceinline__ void load_shallow_all(std::integer_sequence<int, I...>) const {
    (load_shallow<I>(), ...);
  }
  template <int... I>
  __device__ __forceinline__ void load_deep_all(std::integer_sequence<int, I...>) const {
    (load_deep<I>(), ...);
  }
  __device__ __forceinline__ const lds_u8* a_buf(int s) const { return smem + (s % SA) * OP_BYTES; }
  __device__ __forceinline__ const lds_u8* b_buf(int s) const {
    return smem + B_BASE + (s % SB) * OP_BYTES;
  }
};

// MFMA number IDX (block i = IDX/4, j = IDX%4) of a k-step, followed by its
// share of the memory instructions, then a scheduling barrier so that the
// exact order is kept.  bf16 (four k-steps): MFMAs 0..7 of an early k-step
// read the next k-step's fragments; the 16 direct loads of the pending
// slices go one per four MFMAs over the whole slice -- MFMAs 8, 10, 12, 14
// of k-steps 0 and 1 the shallow operand's, of k-step 2 and MFMAs 1, 3, 5, 7
// of the last k-step (before its barrier) the deep operand's -- so that the
// four waves never queue more direct loads than the vector memory path
// drains while one MFMA runs (a wave stalled on a full queue also holds back
// the MFMAs behind the load).  fp8 (two k-steps, each MFMA twice as long):
// k-step 0 carries all of them -- fragment reads and shallow loads in MFMAs
// 0..7, deep loads in 8..15.
template <int KK, int IDX, bool F8, class ST>
__device__ __forceinline__ void kstep_op(const ST& st, const Frags<F8>& cur, Frags<F8>& nxt,
                                         Acc& acc, const lds_u8* As, const lds_u8* Bs,
                                         int kk_next) {
  constexpr int i = IDX / 4, j = IDX % 4;
  if constexpr (F8)
    acc.c[i][j] = mfma32_f8(cur.a[i], cur.b[j], acc.c[i][j]);
  else
    acc.c[i][j] = mfma32(cur.a[i], cur.b[j], acc.c[i][j]);
  constexpr bool last = KK == KSTEPS<F8> - 1;
  if constexpr (!last) {
    if constexpr (IDX < 8) read_frag<IDX>(nxt, As, Bs, st.wm, st.wn, st.lane, kk_next);
    if constexpr (F8) {
      if constexpr (IDX < 8) st.template load_shallow<IDX>();
      else st.template load_deep<IDX - 8>();
    } else {
      constexpr int L = (IDX - 8) / 2;
      if constexpr (IDX >= 8 && IDX % 2 == 0 && KK == 0) st.template load_shallow<L>();
      if constexpr (IDX >= 8 && IDX % 2 == 0 && KK == 1) st.template load_shallow<4 + L>();
      if constexpr (IDX >= 8 && IDX % 2 == 0 && KK == 2) st.template load_deep<L>();
    }
  } else {
    if constexpr (!F8 && IDX < 8 && IDX % 2 == 1) st.template load_deep<4 + IDX / 2>();
    if constexpr (IDX >= 8) read_frag<IDX - 8>(nxt, As, Bs, st.wm, st.wn, st.lane, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int KK, bool F8, class ST, int... IDX>
__device__ __forceinline__ void kstep_ops(const ST& st, const Frags<F8>& cur, Frags<F8>& nxt,
                                          Acc& acc, const lds_u8* As, const lds_u8* Bs,
                                          int kk_next, std::integer_sequence<int, IDX...>) {
  (kstep_op<KK, IDX, F8>(st, cur, nxt, acc, As, Bs, kk_next), ...);
}

// k-step KK of slice kt.  Early k-steps read the next k-step's fragments
// during their first 8 MFMAs and carry direct loads during the other 8
// (the shallow operand's slice kt + 1, the deep operand's slice kt + 2).
// The last k-step runs 8 MFMAs (bf16: with the deep operand's last four
// loads), waits until only the deep operand's loads of this slice are in
// flight (so both operands' slice kt + 1 has landed for this wave) and
// meets the other waves at the workgroup barrier --
// after which slice kt's buffers are free and slice kt + 1 is complete --
// then reads slice kt + 1's first fragments during its last 8 MFMAs.
template <int KK, bool F8, class ST>
__device__ __forceinline__ void mma_kstep(ST& st, Frags<F8>& cur, Frags<F8>& nxt, Acc& acc,
                                          int kt) {
  if constexpr (KK + 1 < KSTEPS<F8>) {
    kstep_ops<KK, F8>(st, cur, nxt, acc, st.a_buf(kt), st.b_buf(kt), KK + 1,
                      std::make_integer_sequence<int, 16>{});
    mma_kstep<KK + 1, F8>(st, nxt, cur, acc, kt);
  } else {
    kstep_ops<KK, F8>(st, cur, nxt, acc, st.a_buf(kt), st.b_buf(kt), 0,
                      std::integer_sequence<int, 0, 1, 2, 3, 4, 5, 6, 7>{});
    wait_vm<LOADS_PER_OP>();
    __syncthreads();
    // slice kt's buffers are free from here on
    st.set_load_shallow(kt + SHALLOW_STAGES);
    st.set_load_deep(kt + DEEP_STAGES);
    kstep_ops<KK, F8>(st, cur, nxt, acc, st.a_buf(kt + 1), st.b_buf(kt + 1), 0,
                      std::integer_sequence<int, 8, 9, 10, 11, 12, 13, 14, 15>{});
  }
}

// Main loop over the k slices [k_begin, k_end) of one tile; PA / PB say
// whether A / B are in the packed operand layout, DEEP_B whether B (else A)
// is the weight operand with the deeper ring, F8 whether both hold e4m3
// codes (packed fp8 layout; Src pointers and strides then count code pairs,
// so a slice is 128 codes deep).  Slices below nk0 take their B rows from
// B0, the others (from slice nk0 on) from B1; A runs straight through.  The
// caller separates two calls on the same LDS with a workgroup barrier.
template <bool PA, bool PB, bool DEEP_B, bool F8 = false>
__device__ __forceinline__ void gemm_mainloop(lds_u8* smem, Acc& acc, const Src& A,
                                              const Src& B0, int nk0, const Src& B1,
                                              int k_begin, int k_end) {
  static_assert(KSTEPS<F8> % 2 == 0, "slices start in the first fragment set");
  Stream<PA, PB, DEEP_B> st;
  st.smem = smem;
  st.lds0 = (uint32_t)(uintptr_t)smem;
  st.A = A;
  st.B0 = B0;
  st.B1 = B1;
  st.nk0 = nk0;
  st.k_begin = k_begin;
  st.nk = k_end - k_begin;
  st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  st.lane = threadIdx.x & 63;
  st.wm = st.wave >> 1;
  st.wn = st.wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc.c[i][j][e] = 0.f;

  // prologue: shallow slice 0, deep slices 0 and 1; shallow slice 1 and deep
  // slice 2 ride on slice 0
  const auto seq = std::make_integer_sequence<int, LOADS_PER_OP>{};
  st.set_load_shallow(0);
  st.load_shallow_all(seq);
  st.set_load_deep(0);
  st.load_deep_all(seq);
  st.set_load_deep(1);
  st.load_deep_all(seq);
  st.set_load_shallow(1);
  st.set_load_deep(2);
  wait_vm<LOADS_PER_OP>();
  __syncthreads();
  Frags<F8> f0, f1;
  const lds_u8* a0 = st.a_buf(0);
  const lds_u8* b0 = st.b_buf(0);
  read_frag<0>(f0, a0, b0, st.wm, st.wn, st.lane, 0);
  read_frag<1>(f0, a0, b0, st.wm, st.wn, st.lane, 0);
  read_frag<2>(f0, a0, b0, st.wm, st.wn, st.lane, 0);
  read_frag<3>(f0, a0, b0, st.wm, st.wn, st.lane, 0);
  read_frag<4>(f0, a0, b0, st.wm, st.wn, st.lane, 0);
  read_frag<5>(f0, a0, b0, st.wm, st.wn, st.lane, 0);
  read_frag<6>(f0, a0, b0, st.wm, st.wn, st.lane, 0);
  read_frag<7>(f0, a0, b0, st.wm, st.wn, st.lane, 0);
  for (int kt = 0; kt < st.nk; ++kt) mma_kstep<0, F8>(st, f0, f1, acc, kt);
  // the re-fetches issued by the last iterations must land before the
  // workgroup can release its LDS
  wait_vm<0>();
}

struct ProjArgs {
  const bf16* h;       // packed bf16 h, or packed e4m3 codes of h (F8)
  // weight sets; a tile takes the set of its row group
  const bf16 *wq[kMaxWeightSets], *wk[kMaxWeightSets], *wv[kMaxWeightSets];
  const bf16 *wg[kMaxWeightSets], *wu[kMaxWeightSets];
  const float* sh;     // F8: dequantisation scale of each h row [n_pad]
  const float* sw[kMaxWeightSets];   // F8: scale of each weight row [3D + 2F], q k v gate up
  const float *qn[kMaxWeightSets], *kn[kMaxWeightSets];
  const float2* rope;  // rows of tokens
  bf16 *q, *k, *vt, *cat;
  RowGroups rg;        // workspace rows -> tokens
  int rows;            // workspace rows covered by tiles
  int n_pad, D, H, F;
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

// acc *= a_scale * b_scale for rowwise-fp8 operands: A row
// wm 128 + 32 i + 8 (e / 4) + 4 (l / 32) + e % 4 takes a_run[i][8 (e / 4) +
// 4 (l / 32) + e % 4] (a_run[i]: the scales of the wave's 32-row run i), B
// row wn 128 + 32 j + l % 32 takes b_scale[32 j + l % 32].
__device__ __forceinline__ void scale_acc(Acc& acc, const float* const (&a_run)[4],
                                          const float* b_scale, int lane) {
  const int hi = lane >> 5, r32 = lane & 31;
  float cs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cs[j] = b_scale[32 * j + r32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 rs = *reinterpret_cast<const float4*>(a_run[i] + 8 * g + 4 * hi);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc.c[i][j][4 * g + 0] *= rs.x * cs[j];
        acc.c[i][j][4 * g + 1] *= rs.y * cs[j];
        acc.c[i][j][4 * g + 2] *= rs.z * cs[j];
        acc.c[i][j][4 * g + 3] *= rs.w * cs[j];
      }
    }
}

// PW: the weights come in the packed operand layout (flux3_weights_pack),
// else in Linear layout.  F8: h and the weights are rowwise e4m3 codes in
// the packed fp8 layout (flux3_weights_quantize_fp8r), the products are
// scaled back by the row scales before the epilogue.
template <bool PW, bool F8>
__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_proj(ProjArgs p) {
  static_assert(PW || !F8, "fp8 weights are always packed");
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[LDS_BYTES];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int qkv_tiles = p.H / 2;
  const int n_n = 3 * qkv_tiles + p.F / 128;
  const int n_m = p.rows / BM;
  int mt, nt;
  tile_coords(blockIdx.x, n_m, n_n, mt, nt);
  const int m0 = mt * BM;
  // the tile's 256 workspace rows lie in one row group (groups start on
  // 256-row boundaries), which also selects the weight set
  const RowMap grp = row_map(p.rg, m0);

  int kind, head0 = 0, hid0 = 0;
  if (nt < 3 * qkv_tiles) {
    kind = nt / qkv_tiles;
    head0 = 2 * (nt % qkv_tiles);
  } else {
    kind = 3;
    hid0 = (nt - 3 * qkv_tiles) * 128;
  }
  const int D = p.D;
  const int Dk = F8 ? D / 2 : D;   // row length in 2-byte units
  // first weight row of 32-row run i of the tile (256 output features)
  auto w_row = [&](int i) -> int {
    if (kind < 3) return head0 * 128 + 32 * i;
    // SwiGLU tiles: each 128-row half holds 64 gate rows then the 64 up rows
    // of the same hidden units, so gate and up land in one lane's registers
    return hid0 + 64 * (i >> 2) + 32 * (i & 1);
  };
  const int ws = grp.w;
  auto w_mat = [&](int i) -> const bf16* {
    if (kind < 3) return kind == 0 ? p.wq[ws] : (kind == 1 ? p.wk[ws] : p.wv[ws]);
    return (i & 3) < 2 ? p.wg[ws] : p.wu[ws];
  };
  auto w_run = [&](int i) -> const bf16* { return w_mat(i) + (size_t)w_row(i) * Dk; };
  Src H, W;   // h is packed, the weights row-major
  H.lo = p.h + (size_t)(m0 + 64 * wave) * Dk;
  H.hi = H.lo;
  H.ld = 8 * Dk;
  W.lo = w_run(2 * wave);
  W.hi = w_run(2 * wave + 1);   // = lo + 32 D: a wave's 64 rows are consecutive rows of one matrix
  W.ld = PW ? 8 * Dk : Dk;
  // Values use C = h . Wv^T (a lane then holds 4 consecutive tokens of one
  // dim, the order of the transposed store).  Queries, keys and SwiGLU use
  // C^T = W . h^T: a lane holds one token and 4 consecutive features per
  // register group, so RoPE pairs are lane-local, the per-head RMS needs one
  // exchange with lane ^ 32, and stores are 8 bytes wide.
  Acc acc;
  if (kind == 2)
    gemm_mainloop<true, PW, true, F8>(smem, acc, H, W, Dk / BK, W, 0, Dk / BK);
  else
    gemm_mainloop<PW, true, false, F8>(smem, acc, W, H, Dk / BK, H, 0, Dk / BK);
  // F8: the row scales multiply the products where the epilogues read them
  // (a scaled copy of the whole accumulator would not fit in registers);
  // sw_kind: the scales of this tile's weight matrix rows, or of the gate
  // rows for SwiGLU (the up rows follow F rows later)
  const float* sw_kind = nullptr;
  if constexpr (F8) sw_kind = p.sw[ws] + (kind < 3 ? kind * D : 3 * D);

  const int r32 = lane & 31, hi = lane >> 5;
  // LDS is free once every wave is past the main loop.  Values and SwiGLU
  // stage their output tile there so that the global stores are whole
  // 16-byte chunks of contiguous rows: staged rows are 256 B (SwiGLU: one
  // token's 128 features) or 512 B (values: one dim's 256 tokens), chunk c
  // of staged row r in slot c ^ (r % 16) or c ^ (r % 32) respectively,
  // which spreads the lanes' 8-byte writes over the banks.  Queries and
  // keys use it for the tile's RoPE rows instead.
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  __syncthreads();
  if (kind < 2) {
    // The RoPE rows of the tile's 256 tokens go to LDS first, by direct
    // loads (2 rows of 512 B per load; rows past the last token repeat it).
    // Chunk c (4 floats = 2 pairs) of row t sits in slot c ^ (t % 32), so the
    // 32 lanes of a read, 32 consecutive tokens at one chunk, hit different
    // banks.  Then per-head RMSNorm + RoPE: this wave holds head head0 + wm
    // for 128 tokens and stores its 4 consecutive dims per register group.
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const float* rope = reinterpret_cast<const float*>(p.rope);
#pragma unroll 8
    for (int it = 0; it < 32; ++it) {
      const int row = wave * 64 + it * 2 + (lane >> 5);
      const int c = (lane & 31) ^ (row & 31);
      const int m = grp.token(m0 + row);
      dma16(reinterpret_cast<const bf16*>(rope + (size_t)m * 2 * kRopePairs + c * 4),
            lds0 + (uint32_t)((wave * 64 + it * 2) * 512));
    }
    wait_vm<0>();
    __syncthreads();
    typedef const __attribute__((address_space(3))) f32x4 lds_f4;
    const float* nw = kind == 0 ? p.qn[ws] : p.kn[ws];
    bf16* dst = (kind == 0 ? p.q : p.k) + (size_t)head0 * p.n_pad * kHeadDim;
    // the norm weights of this lane's 64 dims, loaded once
    float4 nwv[4][4];
    // F8: the scales of the head's 128 weight rows (this wave's head
    // head0 + wm), folded into the norm weights
    const float* swh = F8 ? sw_kind + (head0 + wm) * 128 : nullptr;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        nwv[i][g] = *reinterpret_cast<const float4*>(nw + i * 32 + 8 * g + 4 * hi);
        if constexpr (F8) {
          const float4 sv = *reinterpret_cast<const float4*>(swh + i * 32 + 8 * g + 4 * hi);
          nwv[i][g].x *= sv.x;
          nwv[i][g].y *= sv.y;
          nwv[i][g].z *= sv.z;
          nwv[i][g].w *= sv.w;
        }
      }
    // Output rows go out through the 32 KiB of LDS past the RoPE rows, one
    // register block j at a time: the four waves' 32 tokens x 128 dims
    // (staged row (2 wm + wn) 32 + token, 256 B, 16-byte chunk c in slot
    // c ^ (row % 16)), then stored as whole rows, 1 KiB per instruction.
    // A lane's own 8-byte pieces would touch 32 token rows per instruction.
    constexpr int STAGE = 256 * 512;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = wn * 128 + j * 32 + r32;             // row within the tile
      const bool live = grp.live(m0 + t);
      float ss = 0.f;
      float rs;
      if constexpr (F8) {
        // x = acc * sw[dim] * sh[token]: the RMS over the head's dims of
        // acc * sw, times the token scale; the output factor sh * rs
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 sv = *reinterpret_cast<const float4*>(swh + i * 32 + 8 * g + 4 * hi);
            const float a0 = acc.c[i][j][4 * g] * sv.x, a1 = acc.c[i][j][4 * g + 1] * sv.y;
            const float a2 = acc.c[i][j][4 * g + 2] * sv.z, a3 = acc.c[i][j][4 * g + 3] * sv.w;
            ss += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
          }
        ss += xor_lane(ss, 32);
        const float st = p.sh[m0 + t];
        rs = st / sqrtf(st * st * ss * (1.0f / kHeadDim) + p.eps);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) ss += acc.c[i][j][e] * acc.c[i][j][e];
        ss += xor_lane(ss, 32);
        rs = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + p.eps);
      }
      const int srow = (2 * wm + wn) * 32 + r32;
      // all of the token's RoPE chunks first: a read placed after a staging
      // write would wait for it
      f32x4 csv[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = i * 32 + 8 * g + 4 * hi;
          csv[i][g] = *(lds_f4*)(smem + t * 512 + (((d0 >> 2) ^ (t & 31)) << 4));
        }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = i * 32 + 8 * g + 4 * hi;          // 4 consecutive dims = 2 pairs
          const float4 wv = nwv[i][g];
          const f32x4 cs = csv[i][g];                      // cos0 sin0 cos1 sin1
          const float x0 = acc.c[i][j][4 * g + 0] * rs * wv.x;
          const float x1 = acc.c[i][j][4 * g + 1] * rs * wv.y;
          const float x2 = acc.c[i][j][4 * g + 2] * rs * wv.z;
          const float x3 = acc.c[i][j][4 * g + 3] * rs * wv.w;
          bf16x4 o;
          o[0] = f2bf(live ? x0 * cs.x - x1 * cs.y : 0.f);
          o[1] = f2bf(live ? x0 * cs.y + x1 * cs.x : 0.f);
          o[2] = f2bf(live ? x2 * cs.z - x3 * cs.w : 0.f);
          o[3] = f2bf(live ? x2 * cs.w + x3 * cs.z : 0.f);
          *(lds_bf16x4*)(smem + STAGE + srow * 256 + (((d0 >> 3) ^ (srow & 15)) << 4) + 8 * hi) = o;
        }
      __syncthreads();
      // 128 staged rows; wave w stores rows 32 w .. 32 w + 31, 4 per instruction
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = wave * 32 + it * 4 + (lane >> 4), c = lane & 15;
        const u32x4 v = *(lds_u32x4*)(smem + STAGE + row * 256 + ((c ^ (row & 15)) << 4));
        const int run = row >> 5;                        // 2 head + token half
        const int tok = m0 + (run & 1) * 128 + j * 32 + (row & 31);
        *reinterpret_cast<u32x4*>(dst + ((size_t)(run >> 1) * p.n_pad + tok) * kHeadDim + c * 8) = v;
      }
      if (j < 3) __syncthreads();   // staging free for the next block
    }
  } else if (kind == 2) {
    // values, transposed: staged as [head][dim][256 token positions]
    float swj[4] = {1.f, 1.f, 1.f, 1.f};   // F8: scales of the lane's dim rows
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) swj[j] = sw_kind[head0 * 128 + wn * 128 + j * 32 + r32];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int mb = wm * 128 + i * 32 + 8 * g + 4 * hi;   // first of 4 tokens, tile-local
        const int pos = vt_pos(mb);
        float4 stv = make_float4(1.f, 1.f, 1.f, 1.f);      // F8: the 4 tokens' scales
        if constexpr (F8) stv = *reinterpret_cast<const float4*>(p.sh + m0 + mb);
        const float st[4] = {stv.x, stv.y, stv.z, stv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = wn * 128 + j * 32 + r32;             // head-local dim row
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = F8 ? acc.c[i][j][4 * g + e] * (st[e] * swj[j]) : acc.c[i][j][4 * g + e];
            v[e] = f2bf(grp.live(m0 + mb + e) ? a : 0.f);
          }
          *(lds_bf16x4*)(smem + r * 512 + (((pos >> 3) ^ (r & 31)) << 4) + (pos & 7) * 2) = v;
        }
      }
    }
    __syncthreads();
    // 256 rows (2 heads x 128 dims) of 512 B; a store covers 2 rows
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
      const int row = wave * 64 + it * 2 + (lane >> 5), chunk = lane & 31;
      const u32x4 v = *(lds_u32x4*)(smem + row * 512 + ((chunk ^ (row & 31)) << 4));
      bf16* dst = p.vt + ((size_t)(head0 + (row >> 7)) * kHeadDim + (row & 127)) * p.n_pad + m0 +
                  chunk * 8;
      *reinterpret_cast<u32x4*>(dst) = v;
    }
  } else {
    // SwiGLU: register blocks 0,1 are gate rows, 2,3 the matching up rows;
    // staged as [token][128 hidden units]
    // F8: scales of the lane's gate and up rows (hidden units
    // hid0 + 64 wm + 32 i + 8 g + 4 hi + e)
    float4 sgv[2][4], suv[2][4];
    if constexpr (F8) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float* sg = sw_kind + hid0 + 64 * wm + 32 * i + 8 * g + 4 * hi;
          sgv[i][g] = *reinterpret_cast<const float4*>(sg);
          suv[i][g] = *reinterpret_cast<const float4*>(sg + p.F);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = wn * 128 + j * 32 + r32;
      const bool live = grp.live(m0 + t);
      const float st = F8 ? p.sh[m0 + t] : 1.f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float gt = acc.c[i][j][4 * g + e], up = acc.c[i + 2][j][4 * g + e];
            if constexpr (F8) {
              const float sg[4] = {sgv[i][g].x, sgv[i][g].y, sgv[i][g].z, sgv[i][g].w};
              const float su[4] = {suv[i][g].x, suv[i][g].y, suv[i][g].z, suv[i][g].w};
              gt *= sg[e] * st;
              up *= su[e] * st;
            }
            const float a = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
            o[e] = f2bf(live ? a : 0.f);
          }
          const int chunk = 8 * wm + 4 * i + g;
          *(lds_bf16x4*)(smem + t * 256 + ((chunk ^ (t & 15)) << 4) + 8 * hi) = o;
        }
    }
    __syncthreads();
    // 256 token rows of 256 B; a store covers 4 rows, each 16-byte chunk to
    // its slot of the packed concatenation
    const int ldc = D + p.F;
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int t = wave * 64 + it * 4 + (lane >> 4), chunk = lane & 15;
      const u32x4 v = *(lds_u32x4*)(smem + t * 256 + ((chunk ^ (t & 15)) << 4));
      bf16* dst = p.cat + packed_index(m0 + t, D + hid0 + chunk * 8, ldc);
      *reinterpret_cast<u32x4*>(dst) = v;
    }
  }
}

// One sub-round of K4's tail: tail tiles [first, first + tiles), each cut
// into `pieces` ranges of k slices.
struct TailRound {
  int first, tiles, pieces;
};

struct OutArgs {
  const bf16* cat;     // packed bf16 [o | act], or its packed e4m3 codes (F8)
  // weight sets; a tile takes the set of its row group
  const bf16 *wo[kMaxWeightSets], *wd[kMaxWeightSets];
  const float* scat;   // F8: scale of each cat row [n_pad]
  const float* sw[kMaxWeightSets];   // F8: scale of each row of [wo | wd] [D]
  float* x;            // rows of tokens
  const float* mod;
  float* part;       // split-tile partial sums: 2 slots of BM x BN fp32 per workgroup
  SegTable segs;     // tokens -> segments (modulation rows)
  RowGroups rg;      // workspace rows -> tokens
  int rows;          // workspace rows covered by tiles
  int n_pad, D, F;
  int nk, nk0;       // k slices of a tile, of them from wo
  int groups;        // persistent workgroups G
  int dp_rounds;     // whole-tile rounds before the split tail
  int tail;          // tiles left to the k-piece sub-rounds (0: none)
  TailRound tr0, tr1;   // the sub-rounds (tr1.tiles == 0: one sub-round)
};

// gate_s row of the segment holding token m.
__device__ __forceinline__ const float* gate_row(const OutArgs& p, int m) {
  return p.mod + (size_t)seg_of(p.segs, m) * 3 * p.D + 2 * p.D;
}

// x += gate_s * acc for row block i of a wave (32 rows x 128 columns).
// Lane l holds column l % 32 of each 32-column block j and rows
// 8 (e / 4) + 4 (l / 32) + e % 4, e < 16 (workspace rows of the tile's row
// group grp; each live one is the x row of its token).  Every load is issued
// before the first store and none sits behind a branch: padding rows are
// clamped to the group's last token for the loads, and only the stores are
// predicated.  When the wave's 128 rows lie in one segment (gate_one !=
// null) its gate values are read once per tile.
__device__ __forceinline__ void out_rows(const OutArgs& p, const f32x16 (&v)[4], int i, int m0,
                                         int n0, int wm, int wn, int lane,
                                         const float* gate_one, const RowMap& grp) {
  const int D = p.D;
  const int mb = m0 + wm * 128 + i * 32 + 4 * (lane >> 5);
  const int nb = n0 + wn * 128 + (lane & 31);
  float xv[16][4];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int m = grp.token(mb + 8 * (e >> 2) + (e & 3));
    const float* xr = p.x + (size_t)m * D + nb;
#pragma unroll
    for (int j = 0; j < 4; ++j) xv[e][j] = xr[32 * j];
  }
  float gv[4];
  if (gate_one) {
#pragma unroll
    for (int j = 0; j < 4; ++j) gv[j] = gate_one[nb + 32 * j];
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int r = mb + 8 * (e >> 2) + (e & 3);
    const int m = grp.token(r);
    if (!gate_one) {
      const float* g = gate_row(p, m) + nb;
#pragma unroll
      for (int j = 0; j < 4; ++j) gv[j] = g[32 * j];
    }
    if (grp.live(r)) {
      float* xr = p.x + (size_t)m * D + nb;
#pragma unroll
      for (int j = 0; j < 4; ++j) xr[32 * j] = xv[e][j] + gv[j] * v[j][e];
    }
  }
}

// The gate row shared by all 128 rows of wave row-block wm, or null when
// they straddle a segment boundary.
__device__ __forceinline__ const float* wave_gate(const OutArgs& p, int m0, int wm,
                                                  const RowMap& grp) {
  const int first = grp.token(m0 + wm * 128), last = grp.token(m0 + wm * 128 + 127);
  const int s = seg_of(p.segs, first);
  return s == seg_of(p.segs, last) ? p.mod + (size_t)s * 3 * p.D + 2 * p.D : nullptr;
}

// x += gate_s * acc for the tile's live rows.
__device__ __forceinline__ void out_epilogue(const OutArgs& p, const Acc& acc, int m0, int n0,
                                             int wm, int wn, int lane, const RowMap& grp) {
  const float* g = wave_gate(p, m0, wm, grp);
#pragma unroll
  for (int i = 0; i < 4; ++i) out_rows(p, acc.c[i], i, m0, n0, wm, wn, lane, g, grp);
}

// Partial slot layout: float4 q = 4 (4 i + j) + g of a lane holds
// acc.c[i][j][4g .. 4g + 3] (4 consecutive rows of one column); lane l of
// wave w keeps it at float4 index (64 w + q) 64 + l, so each store or load
// instruction moves 1 KiB contiguously.
__device__ __forceinline__ float4* slot_base(const OutArgs& p, int slot) {
  return reinterpret_cast<float4*>(p.part + (size_t)slot * BM * BN);
}

template <bool PW, bool F8>
__device__ __forceinline__ void out_tile_ptrs(const OutArgs& p, int m0, int n0, int wave, int ws,
                                              Src& A, Src& B0, Src& B1) {
  // row lengths in 2-byte units
  const int D = F8 ? p.D / 2 : p.D, F = F8 ? p.F / 2 : p.F, ldc = D + F;
  A.lo = p.cat + (size_t)(m0 + 64 * wave) * ldc;   // packed
  A.hi = A.lo;
  A.ld = 8 * ldc;
  B0.lo = p.wo[ws] + (size_t)(n0 + 64 * wave) * D;
  B0.hi = B0.lo + (size_t)32 * D;
  B0.ld = PW ? 8 * D : D;
  B1.lo = p.wd[ws] + (size_t)(n0 + 64 * wave) * F;
  B1.hi = B1.lo + (size_t)32 * F;
  B1.ld = PW ? 8 * F : F;
}

// Work split of K4 over G persistent workgroups.  Tiles are numbered in the
// XCD-grouped order of tile_coords.  The first dp_rounds * G of them go
// whole, G at a time (the workgroups of one XCD then walk the same k
// slices of neighbouring tiles together and share them in L2).  The `tail`
// tiles left, when they would leave over a set share of a round idle, run
// as one or two sub-rounds of k pieces: sub-round s cuts tail tiles [first,
// first + tiles) into `pieces` equal k ranges, and its item i < tiles *
// pieces -- piece i / tiles of tail tile first + i % tiles -- runs on the
// workgroup of range index i (range_of_block), so each XCD's workgroups run
// one k range of neighbouring tiles in step and still share slices in L2.
// Item i leaves its partial tile in slot s G + i; the fixup kernel sums a
// tile's pieces in k order and applies the epilogue.  Tail tiles are taken
// in increasing linear index (tail_lin), which keeps them neighbours too.
// F8: cat and the weights are rowwise e4m3 codes in the packed fp8 layout;
// every product tile is scaled back by the row scales as soon as its main
// loop ends, so whole tiles, partial tiles and the fixup see plain sums.
template <bool PW, bool F8>
__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_out(OutArgs p) {
  static_assert(PW || !F8, "fp8 weights are always packed");
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[LDS_BYTES];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_n = p.D / BN;
  const int n_m = p.rows / BM;
  const int n_tiles = n_m * n_n;
  const int nk = p.nk;
  const int G = p.groups;
  const int tile0 = p.dp_rounds * G;
  const int v = range_of_block(blockIdx.x, G);
  // one loop over the work items -- whole tiles, then this workgroup's item
  // of each tail sub-round -- so that the main loop is instantiated once
  int r = 0, sr = 0;
  bool first = true;
  for (;;) {
    int mt, nt, kb = 0, ke = nk, slot = -1;
    if (r < p.dp_rounds && r * G + (int)blockIdx.x < n_tiles) {
      tile_coords(r * G + blockIdx.x, n_m, n_n, mt, nt);
      ++r;
    } else {
      r = p.dp_rounds;
      if (sr == 0 && v >= p.tr0.tiles * p.tr0.pieces) sr = 1;
      if (sr == 1 && v >= p.tr1.tiles * p.tr1.pieces) sr = 2;
      if (sr == 2) break;
      const TailRound tr = sr == 0 ? p.tr0 : p.tr1;
      const int piece = v / tr.tiles;
      lin_coords(tail_lin(tr.first + v % tr.tiles, n_tiles, tile0), n_m, n_n, mt, nt);
      kb = piece * nk / tr.pieces;
      ke = (piece + 1) * nk / tr.pieces;
      slot = sr * G + v;
      ++sr;
    }
    const RowMap grp = row_map(p.rg, mt * BM);
    Src A, B0, B1;
    out_tile_ptrs<PW, F8>(p, mt * BM, nt * BN, wave, grp.w, A, B0, B1);
    if (!first) __syncthreads();   // the previous item's LDS reads are done
    first = false;
    Acc acc;
    gemm_mainloop<true, PW, true, F8>(smem, acc, A, B0, p.nk0, B1, kb, ke);
    if constexpr (F8) {
      const float* a0 = p.scat + mt * BM + wm * 128;
      const float* const a_run[4] = {a0, a0 + 32, a0 + 64, a0 + 96};
      scale_acc(acc, a_run, p.sw[grp.w] + nt * BN + wn * 128, lane);
    }
    if (slot < 0) {
      out_epilogue(p, acc, mt * BM, nt * BN, wm, wn, lane, grp);
    } else {
      float4* dst = slot_base(p, slot) + (size_t)wave * 64 * 64 + lane;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16& c = acc.c[i][j];
            dst[(size_t)(4 * (4 * i + j) + g) * 64] =
                make_float4(c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]);
          }
    }
  }
}

constexpr int FIX_SPLIT = 16;   // fixup workgroups per split tile

// Sums the k pieces of every tail tile in k order and applies the
// epilogue; FIX_SPLIT workgroups share a tile.  A thread takes the float4s
// of four neighbouring lanes of one accumulator group -- 4 rows x 4
// consecutive columns, 64 contiguous bytes of a slot -- so that it updates x
// with float4 accesses; x and gate are loaded before the partials are
// summed.
__global__ __launch_bounds__(NTHREADS) void k_gemm_out_fixup(OutArgs p) {
  const int n_n = p.D / BN;
  const int n_m = p.rows / BM;
  const int tt = blockIdx.x / FIX_SPLIT, chunk = blockIdx.x % FIX_SPLIT;
  const bool second = p.tr1.tiles > 0 && tt >= p.tr1.first;
  const TailRound tr = second ? p.tr1 : p.tr0;
  const int slot0 = (second ? p.groups : 0) + (tt - tr.first);

  // float4 f0 .. f0 + 3 of the slot: lanes l0 .. l0 + 3 of group (w, q)
  const int f0 = 4 * (chunk * NTHREADS + threadIdx.x);
  const int l0 = f0 & 63, q = (f0 >> 6) & 63, w = f0 >> 12;
  const int ij = q >> 2, g = q & 3, ii = ij >> 2, jj = ij & 3;
  int mt, nt;
  lin_coords(tail_lin(tt, n_m * n_n, p.dp_rounds * p.groups), n_m, n_n, mt, nt);
  const int m = mt * BM + (w >> 1) * 128 + ii * 32 + 8 * g + 4 * (l0 >> 5);   // workspace row
  const int n = nt * BN + (w & 1) * 128 + jj * 32 + (l0 & 31);
  const RowMap grp = row_map(p.rg, mt * BM);
  float4 xv[4], gv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int mr = grp.token(m + r);
    xv[r] = *reinterpret_cast<const float4*>(p.x + (size_t)mr * p.D + n);
    gv[r] = *reinterpret_cast<const float4*>(gate_row(p, mr) + n);
  }
  float4 sum[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) sum[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int piece = 0; piece < tr.pieces; ++piece) {
    const float4* src = slot_base(p, slot0 + piece * tr.tiles) + f0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 x = src[u];
      sum[u].x += x.x;
      sum[u].y += x.y;
      sum[u].z += x.z;
      sum[u].w += x.w;
    }
  }
  // sum[u] holds column n + u, rows m .. m + 3
  const float c[4][4] = {{sum[0].x, sum[1].x, sum[2].x, sum[3].x},
                         {sum[0].y, sum[1].y, sum[2].y, sum[3].y},
                         {sum[0].z, sum[1].z, sum[2].z, sum[3].z},
                         {sum[0].w, sum[1].w, sum[2].w, sum[3].w}};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (!grp.live(m + r)) continue;
    float4 o = xv[r];
    o.x += gv[r].x * c[r][0];
    o.y += gv[r].y * c[r][1];
    o.z += gv[r].z * c[r][2];
    o.w += gv[r].w * c[r][3];
    *reinterpret_cast<float4*>(p.x + (size_t)grp.token(m + r) * p.D + n) = o;
  }
}

// Linear-layout [R][K] bf16 matrix -> the packed operand layout, one thread
// per 16-byte chunk (8 consecutive k-values of one row).
__global__ __launch_bounds__(256) void k_pack_rows(const bf16* __restrict__ in,
                                                   bf16* __restrict__ out, int R, int K) {
  const int64_t cpr = K / 8;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)R * cpr) return;
  const int64_t r = id / cpr;
  const int k = (int)(id - r * cpr) * 8;
  *reinterpret_cast<u32x4*>(out + packed_index(r, k, K)) =
      *reinterpret_cast<const u32x4*>(in + r * K + k);
}

// ---------------------------------------------------------------------------
// Linears around the block stack (input projections, output projection):
// C[M][N] = A[M][K] W[N][K]^T with A in the packed layout (rows up to m_pad,
// the padding zero) and W Linear or packed (rows up to n_pad).  A tile's k
// slices may be cut into S equal pieces, each its own workgroup, when the
// tiles alone would leave most CUs idle (the 240 x 20480 text projection
// has 12 tiles); pieces store fp32 partial tiles and k_split_reduce adds them
// in piece order.  With S = 1 the tile is stored straight to C.
struct SplitArgs {
  const bf16* a;
  const bf16* w;
  float* part;    // [S][m_pad][n_pad] when S > 1
  float* out;     // C rows m < M, columns n < N, row stride ldo, when S == 1
  int M, m_pad, N, n_pad, K, S, ldo;
};

template <bool PB>
__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_split(SplitArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[LDS_BYTES];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_m = p.m_pad / BM, n_n = p.n_pad / BN, tiles = n_m * n_n;
  const int piece = blockIdx.x / tiles;
  int mt, nt;
  tile_coords(blockIdx.x - piece * tiles, n_m, n_n, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int nk = p.K / BK;
  const int kb = (int)((int64_t)nk * piece / p.S), ke = (int)((int64_t)nk * (piece + 1) / p.S);
  Src A, B;
  A.lo = p.a + (size_t)(m0 + 64 * wave) * p.K;
  A.hi = A.lo;
  A.ld = 8 * p.K;
  B.lo = p.w + (size_t)(n0 + 64 * wave) * p.K;
  B.hi = B.lo + (size_t)32 * p.K;
  B.ld = PB ? 8 * p.K : p.K;
  Acc acc;
  gemm_mainloop<true, PB, true>(smem, acc, A, B, nk, B, kb, ke);
  const int nb = n0 + wn * 128 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (p.S == 1) {
        if (m >= p.M) continue;
        float* row = p.out + (size_t)m * p.ldo;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (nb + 32 * j < p.N) row[nb + 32 * j] = acc.c[i][j][e];
      } else {
        float* row = p.part + ((size_t)piece * p.m_pad + m) * p.n_pad;
#pragma unroll
        for (int j = 0; j < 4; ++j) row[nb + 32 * j] = acc.c[i][j][e];
      }
    }
}

// C[m][n] = sum over pieces, in piece order; one thread per float4 of C.
__global__ __launch_bounds__(256) void k_split_reduce(SplitArgs p) {
  const int n4 = p.N / 4;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)p.M * n4) return;
  const int m = (int)(id / n4), n = (int)(id - (int64_t)m * n4) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < p.S; ++s) {
    const float4 v =
        *reinterpret_cast<const float4*>(p.part + ((size_t)s * p.m_pad + m) * p.n_pad + n);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<float4*>(p.out + (size_t)m * p.ldo + n) = acc;
}

// Rows [0, M) of a row-major [M][K] fp32 or bf16 matrix -> packed bf16
// [m_pad][K] (fp32 rounded to nearest even), rows [M, m_pad) zero; one
// thread per 8-value chunk.
template <bool F32>
__global__ __launch_bounds__(256) void k_pack_input(const void* __restrict__ in,
                                                    bf16* __restrict__ out, int M, int m_pad,
                                                    int K) {
  const int64_t cpr = K / 8;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)m_pad * cpr) return;
  const int64_t r = id / cpr;
  const int k = (int)(id - r * cpr) * 8;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (r < M) {
    if constexpr (F32) {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(in) + r * K + k);
      const float4 a = src[0], b = src[1];
      bf16x8 h;
      h[0] = f2bf(a.x); h[1] = f2bf(a.y); h[2] = f2bf(a.z); h[3] = f2bf(a.w);
      h[4] = f2bf(b.x); h[5] = f2bf(b.y); h[6] = f2bf(b.z); h[7] = f2bf(b.w);
      v = *reinterpret_cast<const u32x4*>(&h);
    } else {
      v = *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(in) + r * K + k);
    }
  }
  *reinterpret_cast<u32x4*>(out + packed_index(r, k, K)) = v;
}

}  // namespace

hipError_t launch_pack_rows(const void* in, void* out, int R, int K, hipStream_t s) {
  const int64_t chunks = (int64_t)R * (K / 8);
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_rows, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                     static_cast<const bf16*>(in), static_cast<bf16*>(out), R, K);
  return hipGetLastError();
}

hipError_t launch_pack_input(const void* in, bool in_fp32, void* out, int M, int m_pad, int K,
                             hipStream_t s) {
  const int64_t chunks = (int64_t)m_pad * (K / 8);
  if (chunks == 0) return hipSuccess;
  const dim3 grid((unsigned)((chunks + 255) / 256));
  if (in_fp32)
    hipLaunchKernelGGL(k_pack_input<true>, grid, dim3(256), 0, s, in, static_cast<bf16*>(out), M,
                       m_pad, K);
  else
    hipLaunchKernelGGL(k_pack_input<false>, grid, dim3(256), 0, s, in, static_cast<bf16*>(out), M,
                       m_pad, K);
  return hipGetLastError();
}

hipError_t launch_gemm_split(const SplitGemm& g, hipStream_t s) {
  SplitArgs p;
  p.a = static_cast<const bf16*>(g.a);
  p.w = static_cast<const bf16*>(g.w);
  p.part = g.part;
  p.out = g.out;
  p.M = g.M;
  p.m_pad = g.m_pad;
  p.N = g.N;
  p.n_pad = g.n_pad;
  p.K = g.K;
  p.S = g.S;
  p.ldo = g.ldo;
  if (g.M == 0) return hipSuccess;
  const unsigned grid = (unsigned)((g.m_pad / BM) * (g.n_pad / BN) * g.S);
  if (g.w_packed)
    hipLaunchKernelGGL(k_gemm_split<true>, dim3(grid), dim3(NTHREADS), 0, s, p);
  else
    hipLaunchKernelGGL(k_gemm_split<false>, dim3(grid), dim3(NTHREADS), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.S == 1) return e;
  const int64_t n = (int64_t)g.M * (g.N / 4);
  hipLaunchKernelGGL(k_split_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm_proj(const BlockShape& bs, const WeightSets& sets,
                            const float* rope, const WsPtrs& ws, float eps,
                            hipStream_t s) {
  if (!rows_valid(bs) || sets.n < 1) return hipErrorInvalidValue;
  const BlockWeightsDev& w = sets.w[0];   // layout flags shared by every set
  ProjArgs p;
  p.h = static_cast<const bf16*>(w.fp8 ? ws.h8 : ws.h);
  p.sh = ws.sh;
  for (int i = 0; i < kMaxWeightSets; ++i) {
    const BlockWeightsDev& v = sets.w[i < sets.n ? i : 0];
    p.sw[i] = v.s_proj;
    p.wq[i] = static_cast<const bf16*>(v.wq);
    p.wk[i] = static_cast<const bf16*>(v.wk);
    p.wv[i] = static_cast<const bf16*>(v.wv);
    p.wg[i] = static_cast<const bf16*>(v.w_gate);
    p.wu[i] = static_cast<const bf16*>(v.w_up);
    p.qn[i] = v.q_norm;
    p.kn[i] = v.k_norm;
  }
  p.rope = reinterpret_cast<const float2*>(rope);
  p.q = static_cast<bf16*>(ws.q);
  p.k = static_cast<bf16*>(ws.k);
  p.vt = static_cast<bf16*>(ws.vt);
  p.cat = static_cast<bf16*>(ws.cat);
  p.rg = bs.rg;
  p.rows = bs.rows;
  p.n_pad = bs.n_pad;
  p.D = bs.D;
  p.H = bs.H;
  p.F = bs.F;
  p.eps = eps;
  const int n_n = 3 * (bs.H / 2) + bs.F / 128;
  const int n_m = bs.rows / BM;
  if (w.fp8)
    hipLaunchKernelGGL((k_gemm_proj<true, true>), dim3(n_m * n_n), dim3(NTHREADS), 0, s, p);
  else if (w.packed)
    hipLaunchKernelGGL((k_gemm_proj<true, false>), dim3(n_m * n_n), dim3(NTHREADS), 0, s, p);
  else
    hipLaunchKernelGGL((k_gemm_proj<false, false>), dim3(n_m * n_n), dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

// Persistent workgroups for the split kernels: one per CU of the current
// device, at most kMaxSplitGroups (the workspace's partial slots).  Queried
// on every call; the library keeps no state across calls.
int stream_k_groups() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return kMaxSplitGroups;
  return cus < kMaxSplitGroups ? cus : kMaxSplitGroups;
}

hipError_t launch_gemm_out(const BlockShape& bs, const WeightSets& sets,
                           const WsPtrs& ws, float* x, const float* mod,
                           const SegTableHost& segs, hipStream_t s) {
  if (!rows_valid(bs) || sets.n < 1) return hipErrorInvalidValue;
  const BlockWeightsDev& w = sets.w[0];   // layout flags shared by every set
  OutArgs p;
  p.cat = static_cast<const bf16*>(w.fp8 ? ws.cat8 : ws.cat);
  for (int i = 0; i < kMaxWeightSets; ++i) {
    const BlockWeightsDev& v = sets.w[i < sets.n ? i : 0];
    p.wo[i] = static_cast<const bf16*>(v.wo);
    p.wd[i] = static_cast<const bf16*>(v.w_down);
    p.sw[i] = v.s_out;
  }
  p.scat = ws.scat;
  // a slice is 64 bf16 values or 128 fp8 codes deep
  const int slice = w.fp8 ? 2 * BK : BK;
  p.nk = (bs.D + bs.F) / slice;
  p.nk0 = bs.D / slice;
  p.x = x;
  p.mod = mod;
  p.part = static_cast<float*>(ws.part);
  for (int i = 0; i < kMaxSegs; ++i) p.segs.start[i] = segs.start[i];
  p.segs.n = segs.n;
  p.rg = bs.rg;
  p.rows = bs.rows;
  p.n_pad = bs.n_pad;
  p.D = bs.D;
  p.F = bs.F;
  p.groups = stream_k_groups();
  const int n_tiles = (bs.rows / BM) * (bs.D / BN);
  const int G = p.groups;
  p.dp_rounds = n_tiles / G;
  p.tail = n_tiles % G;
  // The leftover tiles run as one more round of whole tiles unless they
  // fill little enough of a round (threshold below); then as k-piece
  // sub-rounds.  Measured per launch, sub-rounds against a whole round:
  // bf16 8432 tokens (140 tiles, 55% of a round) 567 us against ~650 (an
  // even stream-K split of the same tail, whose ranges start at scattered k
  // offsets and share nothing in L2: 607); 4096 tokens (75%) 300 against
  // 303; 4336 tokens (80%) 320 against 306; 240 tokens (12 tiles) 51 (the
  // stream-K split: 67).  fp8 slices are half as long and favour whole
  // tiles sooner: 8432 tokens 318 split, 304 whole.  Without a partial-slot
  // region (ws.part null) every tile runs whole.
  const int split_pct = w.fp8 ? 45 : 78;
  if (p.tail * 100 >= G * split_pct || ws.part == nullptr || G < 2) {
    p.dp_rounds += p.tail > 0 ? 1 : 0;
    p.tail = 0;
  }
  // Sub-round plan: pieces = max(2, G / tiles left), as many tiles as that
  // many pieces fit in G items, at least 4 k slices a piece.  Two sub-rounds
  // always suffice: after the first (pieces 2, G / 2 tiles) fewer than G / 2
  // tiles are left, and G / left pieces of each fit.
  p.tr0 = TailRound{0, 0, 1};
  p.tr1 = TailRound{0, 0, 1};
  int left = p.tail, first = 0;
  for (int sr = 0; sr < 2 && left > 0; ++sr) {
    const int pieces = std::min(std::max(2, G / left), std::max(1, p.nk / 4));
    const int tiles = std::min(left, G / pieces);
    (sr == 0 ? p.tr0 : p.tr1) = TailRound{first, tiles, pieces};
    first += tiles;
    left -= tiles;
  }
  if (left > 0) {   // not reached with the plan above; run whole instead
    p.dp_rounds += 1;
    p.tail = 0;
    p.tr0 = TailRound{0, 0, 1};
    p.tr1 = TailRound{0, 0, 1};
  }
  if (w.fp8)
    hipLaunchKernelGGL((k_gemm_out<true, true>), dim3(G), dim3(NTHREADS), 0, s, p);
  else if (w.packed)
    hipLaunchKernelGGL((k_gemm_out<true, false>), dim3(G), dim3(NTHREADS), 0, s, p);
  else
    hipLaunchKernelGGL((k_gemm_out<false, false>), dim3(G), dim3(NTHREADS), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.tail == 0) return e;
  hipLaunchKernelGGL(k_gemm_out_fixup, dim3(p.tail * FIX_SPLIT), dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace flux3
