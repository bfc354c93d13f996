// Host-side launch interface between the C ABI (abi.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace flux3 {

struct RopeLayoutDev {
  int32_t n_text, grid_h, grid_w, n_refs;
  int32_t ref_h[15], ref_w[15];
  double theta, hw_scale;
};

// Rows of one block launch.  Group g's tokens [x_start, x_start + count)
// (rows of x, of the rotary tables and of the segment table) sit at
// workspace rows [ws_start, ws_start + count), ws_start a multiple of 256;
// workspace rows from there up to the next group's start are padding.  Group
// g takes weight set wsel and, in a grouped launch, attends within itself.  A
// plain block is one group with ws_start = x_start = 0 and count = M.
struct RowGroups {
  int32_t ws_start[16], x_start[16], count[16], wsel[16];
  int32_t n;
};

// The plain block's mapping: tokens [0, M) at workspace rows [0, M), set 0.
inline RowGroups one_group(int32_t M) {
  RowGroups g = {};
  g.n = 1;
  g.count[0] = M;
  return g;
}

struct BlockShape {
  int32_t M;       // tokens in this call
  int32_t n_pad;   // M rounded up to 256: row count (stride) of workspace buffers
  int32_t D;       // width
  int32_t H;       // heads
  int32_t F;       // SwiGLU hidden
  int32_t rows = 0;    // workspace rows the GEMMs cover (a multiple of 256, <= n_pad)
  RowGroups rg = {};   // launchers reject a shape whose groups are unset (n == 0)
};

// The row set-up a launcher accepts: 1..16 groups, rows a multiple of 256
// within n_pad.
inline bool rows_valid(const BlockShape& bs) {
  return bs.rg.n >= 1 && bs.rg.n <= 16 && bs.rows >= 0 && bs.rows % 256 == 0 &&
         bs.rows <= bs.n_pad;
}

struct SegTableHost {
  int32_t start[16];
  int32_t n;
};

struct WsPtrs {
  void* h;    // bf16 [n_pad][D]
  void* q;    // bf16 [H][n_pad][128]
  void* k;    // bf16 [H][n_pad][128]
  void* vt;   // bf16 [H][128][n_pad]
  void* cat;  // bf16 [n_pad][D + F]
  void* part; // fp32 [2 kMaxSplitGroups][256 * 256]: split-tile partials of K4 and K3;
              // null: no such region, the split kernels run every tile whole
  // rowwise-fp8 blocks only (packed e4m3 codes, fp32 row scales); they live in
  // buffers that are dead at the time: h8 / sh from K1 to K2, cat8 / scat from
  // the cat quantisation to K4 (over h, q, k, vt once attention is done)
  void* h8;    // [n_pad][D]
  float* sh;   // [n_pad]
  void* cat8;  // [n_pad][D + F]
  float* scat; // [n_pad]
};

// Upper bound on the persistent workgroups of the output GEMM (one
// per CU, at most this many); the workspace holds two partial tiles for each.
constexpr int kMaxSplitGroups = 256;
constexpr size_t kSplitSlotBytes = 256 * 256 * 4;

struct BlockWeightsDev {
  const void *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;
  const float *q_norm, *k_norm;
  bool packed;   // matrices in the packed operand layout
  bool fp8;      // rowwise e4m3 codes in the packed fp8 layout (packed too)
  const float* s_proj;  // fp8: row scales of wq, wk, wv, w_gate, w_up [3D + 2F]
  const float* s_out;   // fp8: row scales of [wo | w_down] [D]
};

// The weight sets of one launch (a group's RowGroups::wsel indexes them);
// all share the layout flags of w[0].
constexpr int kMaxWeightSets = 3;
struct WeightSets {
  BlockWeightsDev w[kMaxWeightSets];
  int n;
};

// Linear-layout [R][K] bf16 (R % 8 == 0, K % 64 == 0) -> packed operand layout.
hipError_t launch_pack_rows(const void* in, void* out, int R, int K, hipStream_t s);

// Rows [0, M) of a row-major fp32 (in_fp32) or bf16 [M][K] matrix -> packed
// bf16 [m_pad][K], padding rows zero (M <= m_pad, m_pad % 8 == 0, K % 64 == 0).
hipError_t launch_pack_input(const void* in, bool in_fp32, void* out, int M, int m_pad, int K,
                             hipStream_t s);

// C[M][N] (fp32, row stride ldo) = A W^T: A packed bf16 [m_pad][K], W bf16
// [n_pad][K] (packed or Linear), m_pad and n_pad multiples of 256, K of 64,
// N of 4.  S > 1 cuts each tile's k slices into S pieces summed through part
// ([S][m_pad][n_pad] fp32) in piece order.
struct SplitGemm {
  const void* a;
  const void* w;
  bool w_packed;
  float* part;
  float* out;
  int M, m_pad, N, n_pad, K, S, ldo;
};
hipError_t launch_gemm_split(const SplitGemm& g, hipStream_t s);

// Timestep path (NEXT-1): distinct timesteps of the used modes first, the
// flow-map target last when present; t_index[mode] indexes t.
struct ModulationShape {
  int32_t D;
  int32_t n_t;         // distinct timesteps of the modes the segments use (1..3)
  int32_t has_target;
  float t[4];
  int32_t t_index[3];
};

struct ModulationWeightsDev {
  const void *w1, *w2, *w1_tgt, *w2_tgt;
  const void* w_mod[3];
  const void* w_final;   // output layer's (shift, scale) linear [2D][D], with final_mod
};

size_t modulation_workspace_floats(int D);
// mod[segment] = (shift, scale, gate) of the segment's mode; with final_mod
// (image mode in use) also the output layer's (shift, scale) from w.w_final.
hipError_t launch_modulation(const ModulationShape& ms, const ModulationWeightsDev& w,
                             const SegTableHost& segs, const int32_t* seg_mode, float* mod,
                             float* ws, hipStream_t s, float* final_mod = nullptr);

// latent += (sigma_next - sigma) v over n fp32 values (n % 4 == 0), with the
// preview x0 = latent - sigma v first when x0 is not null.
hipError_t launch_euler(const float* v, float* latent, float* x0, int64_t n, float sigma,
                        float sigma_next, hipStream_t s);

hipError_t launch_rope_tables(const RopeLayoutDev& lay, float* rope, int64_t n,
                              hipStream_t s);
hipError_t launch_ln_modulate(const BlockShape& bs, const float* x,
                              const float* mod, const SegTableHost& segs,
                              void* h, float eps, hipStream_t s);
// K1 with rowwise-fp8 output: packed e4m3 codes of h [n_pad][D] and the scale
// of each row (rows < M).
hipError_t launch_ln_modulate_f8(const BlockShape& bs, const float* x, const float* mod,
                                 const SegTableHost& segs, void* h8, float* sh, float eps,
                                 hipStream_t s);
// Rowwise e4m3 quantisation of the packed bf16 concatenation [o | act]
// [n_pad][K] into packed fp8 codes and row scales, row blocks of 8 up to
// rows M (K % 128 == 0, K <= kQuantMaxK).
constexpr int kQuantMaxK = 16384;
hipError_t launch_quant_packed_rows(const void* in, void* out, float* scale, int M, int K,
                                    hipStream_t s);
// Rowwise e4m3 quantisation of a Linear-layout bf16 matrix given as two
// column pieces [R][Ka] and [R][Kb] (b may be null with Kb = 0): the codes of
// piece a go to out_a (packed fp8 [R][Ka]), those of b to out_b ([R][Kb]),
// one scale per row over both.  R % 8 == 0, Ka and Kb % 128 == 0,
// Ka + Kb <= kQuantMaxK.
hipError_t launch_quant_weight_rows(const void* a, int Ka, const void* b, int Kb, void* out_a,
                                    void* out_b, float* scale, int R, hipStream_t s);
hipError_t launch_gemm_proj(const BlockShape& bs, const WeightSets& w,
                            const float* rope, const WsPtrs& ws, float eps,
                            hipStream_t s);
// Attention within n_seq sequences of bs.M tokens each, sequence i at
// workspace rows [seq_row[i], seq_row[i] + bs.M) of q, k, v^T and the output
// (n_seq <= 16; one sequence at row 0 for a plain block).
hipError_t launch_attention(const BlockShape& bs, const WsPtrs& ws, const int32_t* seq_row,
                            int n_seq, hipStream_t s);
int stream_k_groups();
hipError_t launch_gemm_out(const BlockShape& bs, const WeightSets& w,
                           const WsPtrs& ws, float* x, const float* mod,
                           const SegTableHost& segs, hipStream_t s);

}  // namespace flux3
