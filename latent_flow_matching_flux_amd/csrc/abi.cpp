// C ABI of libflux3: host-side validation, workspace carving and the
// per-block launch sequence (K1 ln_modulate -> K2 projection GEMM -> K3
// attention -> K4 output GEMM).  Every check runs before the first enqueue,
// so a failing call enqueues nothing.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>

#include <vector>

#include "../../include/flux3.h"
#include "abi_internal.hpp"
#include "kernels.hpp"

namespace {

thread_local char g_detail[512] = "";
std::atomic<int> g_debug_sync{0};   // process-wide; any thread may set it

// Kernel timing records (flux3_profile_*), kept per calling thread.  The
// HIP events of a record are created when its launch is enqueued with
// profiling on, and destroyed by flux3_profile_reset on the same thread.
struct ProfRec {
  int kind;
  hipEvent_t a, b;
  double m, m2;   // tokens; sum of squared sequence lengths (attention work)
};
thread_local bool g_prof_on = false;
thread_local std::vector<ProfRec> g_prof;

hipEvent_t new_event() {
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records the start event of a launch when profiling; returns its index.
// m2 < 0 stands for m * m (one sequence of m tokens).
int prof_begin(int kind, double m, hipStream_t s, double m2 = -1.0) {
  if (!g_prof_on) return -1;
  ProfRec r{kind, new_event(), new_event(), m, m2 < 0 ? m * m : m2};
  if (!r.a || !r.b || hipEventRecord(r.a, s) != hipSuccess) {
    if (r.a) (void)hipEventDestroy(r.a);
    if (r.b) (void)hipEventDestroy(r.b);
    return -1;
  }
  g_prof.push_back(r);
  return (int)g_prof.size() - 1;
}

void prof_end(int idx, hipStream_t s) {
  if (idx >= 0) (void)hipEventRecord(g_prof[idx].b, s);
}

flux3_status fail(flux3_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof g_detail, fmt, ap);
  va_end(ap);
  return s;
}

flux3_status ok() {
  g_detail[0] = '\0';
  return FLUX3_OK;
}

constexpr float kEpsLN = 1e-6f;
constexpr float kEpsRMS = 1e-6f;
constexpr int64_t kRowAlign = 256;     // workspace rows are padded to this
constexpr size_t kBufAlign = 256;      // byte alignment of each workspace buffer
constexpr int64_t kMaxTokens = 1 << 20;
// Caps on the dims, far above the model family's (24 heads, hidden 9216), so
// that the int arithmetic on widths (3 D + 2 F GEMM rows, D + F) stays exact.
constexpr int kMaxHeads = 512;        // width at most 65536
constexpr int kMaxHidden = 1 << 18;   // SwiGLU hidden at most 262144
constexpr int kMaxTextDim = 1 << 18;  // text-encoder feature width at most 262144

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

flux3_status check_dims(const flux3_dims* d) {
  if (!d) return fail(FLUX3_E_INVALID, "dims is NULL");
  if (d->head_dim != 128)
    return fail(FLUX3_E_UNSUPPORTED, "head_dim %d unsupported (must be 128)", d->head_dim);
  if (d->heads < 2 || d->heads % 2 != 0 || d->heads > kMaxHeads)
    return fail(FLUX3_E_UNSUPPORTED, "heads %d unsupported (must be a positive even number, at most %d)",
                d->heads, kMaxHeads);
  if (d->width != d->heads * 128)
    return fail(FLUX3_E_UNSUPPORTED, "width %d != heads*128 (%d)", d->width, d->heads * 128);
  if (d->mlp_hidden <= 0 || d->mlp_hidden % 128 != 0 || d->mlp_hidden > kMaxHidden)
    return fail(FLUX3_E_UNSUPPORTED, "mlp_hidden %d unsupported (positive multiple of 128, at most %d)",
                d->mlp_hidden, kMaxHidden);
  return FLUX3_OK;
}

bool layout_of(const flux3_dims* d, int64_t n, flux3_workspace_layout* L) {
  const int64_t n_pad = (n + kRowAlign - 1) / kRowAlign * kRowAlign;
  const size_t D = (size_t)d->width, F = (size_t)d->mlp_hidden, H = (size_t)d->heads;
  size_t off = 0;
  L->n_pad = n_pad;
  L->h = off;   off = align_up(off + (size_t)n_pad * D * 2, kBufAlign);
  L->q = off;   off = align_up(off + H * (size_t)n_pad * 128 * 2, kBufAlign);
  L->k = off;   off = align_up(off + H * (size_t)n_pad * 128 * 2, kBufAlign);
  L->vt = off;  off = align_up(off + H * 128 * (size_t)n_pad * 2, kBufAlign);
  L->cat = off; off = align_up(off + (size_t)n_pad * (D + F) * 2, kBufAlign);
  L->part = off; off = align_up(off + 2 * (size_t)flux3::kMaxSplitGroups * flux3::kSplitSlotBytes,
                                kBufAlign);
  L->total = off;
  return true;
}

// What a rowwise-fp8 block needs of the dims: the quantiser's row length,
// and the codes and scales of [o | act] within the workspace's h, q, k and vt
// buffers (8 width bytes per padded row).
flux3_status check_fp8_dims(const flux3_dims* d) {
  const int D = d->width, F = d->mlp_hidden;
  if (D + F > flux3::kQuantMaxK)
    return fail(FLUX3_E_UNSUPPORTED, "fp8r weights: width + mlp_hidden %d > %d", D + F,
                flux3::kQuantMaxK);
  if (F >= 7 * D)
    return fail(FLUX3_E_UNSUPPORTED, "fp8r weights: mlp_hidden %d >= 7 width", F);
  return FLUX3_OK;
}

flux3_status check_weights(const flux3_block_weights* w, const char* what, int idx,
                           const flux3_dims* d) {
  if (!w) return fail(FLUX3_E_INVALID, "%s[%d] weights struct is NULL", what, idx);
  const void* ptrs[9] = {w->wq, w->wk, w->wv, w->wo, w->w_gate, w->w_up, w->w_down,
                         w->q_norm, w->k_norm};
  static const char* names[9] = {"wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down",
                                 "q_norm", "k_norm"};
  for (int i = 0; i < 9; ++i) {
    if (!ptrs[i]) return fail(FLUX3_E_INVALID, "%s[%d].%s is NULL", what, idx, names[i]);
    if (!aligned16(ptrs[i]))
      return fail(FLUX3_E_ALIGN, "%s[%d].%s is not 16-byte aligned", what, idx, names[i]);
  }
  if (w->layout != FLUX3_WEIGHTS_LINEAR && w->layout != FLUX3_WEIGHTS_PACKED &&
      w->layout != FLUX3_WEIGHTS_FP8R)
    return fail(FLUX3_E_INVALID, "%s[%d].layout %d is not a FLUX3_WEIGHTS_* value", what, idx,
                w->layout);
  if (w->layout == FLUX3_WEIGHTS_FP8R) {
    if (!w->s_proj || !w->s_out)
      return fail(FLUX3_E_INVALID, "%s[%d]: fp8r weights need s_proj and s_out", what, idx);
    if (!aligned16(w->s_proj) || !aligned16(w->s_out))
      return fail(FLUX3_E_ALIGN, "%s[%d]: s_proj or s_out is not 16-byte aligned", what, idx);
    flux3_status r = check_fp8_dims(d);
    if (r != FLUX3_OK) return r;
  }
  return FLUX3_OK;
}

flux3_status check_segments(const flux3_segment* segs, int32_t n_segs, int64_t n,
                            flux3::SegTableHost* st) {
  if (n_segs < 1 || n_segs > FLUX3_MAX_SEGMENTS)
    return fail(FLUX3_E_SHAPE, "n_segs %d outside [1, %d]", n_segs, FLUX3_MAX_SEGMENTS);
  if (!segs) return fail(FLUX3_E_INVALID, "segs is NULL");
  int64_t pos = 0;
  int prev_mode = 0;
  for (int i = 0; i < n_segs; ++i) {
    const flux3_segment& s = segs[i];
    if (s.mode < FLUX3_MODE_TEXT || s.mode > FLUX3_MODE_REF)
      return fail(FLUX3_E_INVALID, "segment %d has mode %d", i, s.mode);
    if (s.mode < prev_mode)
      return fail(FLUX3_E_SHAPE, "segment %d mode %d after mode %d (order is text, image, reference)",
                  i, s.mode, prev_mode);
    if (s.count <= 0) return fail(FLUX3_E_SHAPE, "segment %d has count %d", i, s.count);
    if (s.start != pos)
      return fail(FLUX3_E_SHAPE, "segment %d starts at %d, expected %lld", i, s.start, (long long)pos);
    pos += s.count;
    prev_mode = s.mode;
    st->start[i] = s.start;
  }
  for (int i = n_segs; i < 16; ++i) st->start[i] = 0;
  st->n = n_segs;
  if (pos != n)
    return fail(FLUX3_E_SHAPE, "segments cover %lld tokens, n_tokens is %lld", (long long)pos,
                (long long)n);
  return FLUX3_OK;
}

flux3_status check_ws(const flux3_dims* d, int64_t n, void* ws, size_t ws_bytes,
                      flux3_workspace_layout* L) {
  layout_of(d, n, L);
  if (!ws) return fail(FLUX3_E_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & (kBufAlign - 1)) != 0)
    return fail(FLUX3_E_ALIGN, "workspace is not %zu-byte aligned", kBufAlign);
  if (ws_bytes < L->total)
    return fail(FLUX3_E_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L->total);
  return FLUX3_OK;
}

flux3::WsPtrs carve(void* ws, const flux3_workspace_layout& L) {
  char* b = static_cast<char*>(ws);
  flux3::WsPtrs p;
  p.h = b + L.h;
  p.q = b + L.q;
  p.k = b + L.k;
  p.vt = b + L.vt;
  p.cat = b + L.cat;
  p.part = b + L.part;
  return p;
}

flux3::BlockWeightsDev dev_weights(const flux3_block_weights& w) {
  flux3::BlockWeightsDev d;
  d.wq = w.wq; d.wk = w.wk; d.wv = w.wv; d.wo = w.wo;
  d.w_gate = w.w_gate; d.w_up = w.w_up; d.w_down = w.w_down;
  d.q_norm = w.q_norm; d.k_norm = w.k_norm;
  d.packed = w.layout == FLUX3_WEIGHTS_PACKED || w.layout == FLUX3_WEIGHTS_FP8R;
  d.fp8 = w.layout == FLUX3_WEIGHTS_FP8R;
  d.s_proj = d.fp8 ? w.s_proj : nullptr;
  d.s_out = d.fp8 ? w.s_out : nullptr;
  return d;
}

flux3_status after_launch(hipError_t e, const char* what, hipStream_t s) {
  if (e != hipSuccess) return fail(FLUX3_E_HIP, "%s launch: %s", what, hipGetErrorString(e));
  if (g_debug_sync.load(std::memory_order_relaxed)) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(FLUX3_E_HIP, "%s execution: %s", what, hipGetErrorString(e));
  }
  return FLUX3_OK;
}

// One block launch sequence (arguments already validated).  `rg` maps workspace rows to tokens: one
// group at rows = tokens for a plain block, one group per segment (each
// starting on a 256-row boundary, with its own weight set and attention over
// its own rows) for a grouped launch of stage-1 blocks; n is the launch's
// token count and rows the workspace rows its GEMM tiles cover.  With split
// false the workspace has no split-partial region (only the buffers before
// `part`); the output GEMM and attention then run their leftover tiles whole
// instead of splitting them.
flux3_status run_block_groups(const flux3_dims* d, const flux3::WeightSets& sets,
                              const flux3::RowGroups& rg, int64_t rows, float* x, int64_t n,
                              const flux3::SegTableHost& st, const float* mod, const float* rope,
                              void* ws, int64_t ws_tokens, hipStream_t s, bool split) {
  flux3_workspace_layout L;
  layout_of(d, ws_tokens, &L);
  flux3::WsPtrs wp = carve(ws, L);
  if (!split) wp.part = nullptr;
  const flux3::BlockWeightsDev& wd = sets.w[0];
  if (wd.fp8) {
    // h's codes and scales in h's buffer (dead until the next block's K1);
    // those of [o | act] from the start of h over q, k and vt, which nothing
    // reads once attention is done (check_fp8_dims keeps them below cat)
    char* base = static_cast<char*>(wp.h);
    const size_t n_pad = (size_t)L.n_pad;
    wp.h8 = base;
    wp.sh = reinterpret_cast<float*>(base + n_pad * (size_t)d->width);
    wp.cat8 = base;
    wp.scat = reinterpret_cast<float*>(
        base + align_up(n_pad * (size_t)(d->width + d->mlp_hidden), kBufAlign));
  }
  flux3::BlockShape bs;
  bs.M = (int32_t)n;
  bs.n_pad = (int32_t)L.n_pad;
  bs.D = d->width;
  bs.H = d->heads;
  bs.F = d->mlp_hidden;
  bs.rows = (int32_t)rows;
  bs.rg = rg;
  flux3_status r;
  const double m = (double)n;
  int pi = prof_begin(FLUX3_K_LN_MODULATE, m, s);
  hipError_t e = wd.fp8 ? flux3::launch_ln_modulate_f8(bs, x, mod, st, wp.h8, wp.sh, kEpsLN, s)
                        : flux3::launch_ln_modulate(bs, x, mod, st, wp.h, kEpsLN, s);
  prof_end(pi, s);
  if ((r = after_launch(e, "ln_modulate", s)) != FLUX3_OK) return r;
  pi = prof_begin(FLUX3_K_GEMM_PROJ, m, s);
  e = flux3::launch_gemm_proj(bs, sets, rope, wp, kEpsRMS, s);
  prof_end(pi, s);
  if ((r = after_launch(e, "gemm_proj", s)) != FLUX3_OK) return r;
  // attention within each group, from the group's first workspace row (a
  // multiple of 256, so the packed output layout shifts by whole row
  // blocks); groups of equal length share a launch, whose units then cover
  // heads x groups
  bool done[16] = {};
  for (int g = 0; g < rg.n; ++g) {
    if (done[g]) continue;
    int32_t rows0[16];
    int n_eq = 0;
    for (int h = g; h < rg.n; ++h)
      if (!done[h] && rg.count[h] == rg.count[g]) {
        rows0[n_eq++] = rg.ws_start[h];
        done[h] = true;
      }
    flux3::BlockShape bg = bs;
    bg.M = rg.count[g];
    pi = prof_begin(FLUX3_K_ATTENTION, (double)bg.M * n_eq, s, (double)bg.M * bg.M * n_eq);
    e = flux3::launch_attention(bg, wp, rows0, n_eq, s);
    prof_end(pi, s);
    if ((r = after_launch(e, "attention", s)) != FLUX3_OK) return r;
  }
  if (wd.fp8) {
    pi = prof_begin(FLUX3_K_QUANT, m, s);
    e = flux3::launch_quant_packed_rows(wp.cat, wp.cat8, wp.scat, rg.n == 1 ? bs.M : bs.rows,
                                        bs.D + bs.F, s);
    prof_end(pi, s);
    if ((r = after_launch(e, "quant_cat", s)) != FLUX3_OK) return r;
  }
  pi = prof_begin(FLUX3_K_GEMM_OUT, m, s);
  e = flux3::launch_gemm_out(bs, sets, wp, x, mod, st, s);
  prof_end(pi, s);
  if ((r = after_launch(e, "gemm_out", s)) != FLUX3_OK) return r;
  return FLUX3_OK;
}

// A plain block on rows [0, n) of x with one weight set.
flux3_status run_block(const flux3_dims* d, const flux3_block_weights& w, float* x, int64_t n,
                       const flux3::SegTableHost& st, const float* mod, const float* rope,
                       void* ws, hipStream_t s, bool split = true) {
  flux3::WeightSets sets;
  sets.w[0] = dev_weights(w);
  sets.n = 1;
  const int64_t rows = (n + kRowAlign - 1) / kRowAlign * kRowAlign;
  return run_block_groups(d, sets, flux3::one_group((int32_t)n), rows, x, n, st, mod, rope, ws, n,
                          s, split);
}


// Validates one stage's modulation inputs for the segments (already
// checked) and fills the launch description.  Nothing is enqueued.
flux3_status prepare_modulation(const flux3_dims* dims, const flux3_modulation_weights* w,
                                const float* t_by_mode, float t_target,
                                const flux3_segment* segs, int32_t n_segs,
                                flux3::ModulationShape* ms, flux3::ModulationWeightsDev* wd,
                                int32_t* seg_mode) {
  const int D = dims->width;
  if (D > 4096) return fail(FLUX3_E_UNSUPPORTED, "modulation supports width <= 4096, got %d", D);
  if (!w) return fail(FLUX3_E_INVALID, "modulation weights struct is NULL");
  if (!t_by_mode) return fail(FLUX3_E_INVALID, "t_by_mode is NULL");
  const void* mats[4] = {w->w1, w->w2, w->w1_tgt, w->w2_tgt};
  static const char* names[4] = {"w1", "w2", "w1_tgt", "w2_tgt"};
  if (t_target != t_target) return fail(FLUX3_E_INVALID, "t_target is NaN");
  const bool target = t_target >= 0.f;
  for (int i = 0; i < (target ? 4 : 2); ++i) {
    if (!mats[i]) return fail(FLUX3_E_INVALID, "%s is NULL", names[i]);
    if (!aligned16(mats[i])) return fail(FLUX3_E_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  if (target && !std::isfinite(t_target)) return fail(FLUX3_E_INVALID, "t_target is not finite");
  // distinct timesteps of the modes in use, in mode order; the target last
  memset(ms, 0, sizeof *ms);
  ms->D = D;
  bool used[3] = {false, false, false};
  for (int i = 0; i < n_segs; ++i) {
    seg_mode[i] = segs[i].mode;
    used[segs[i].mode] = true;
  }
  for (int m = 0; m < 3; ++m) {
    if (!used[m]) continue;
    if (!w->w_mod[m]) return fail(FLUX3_E_INVALID, "w_mod[%d] is NULL but a segment uses mode %d", m, m);
    if (!aligned16(w->w_mod[m])) return fail(FLUX3_E_ALIGN, "w_mod[%d] is not 16-byte aligned", m);
    const float t = t_by_mode[m];
    if (!std::isfinite(t)) return fail(FLUX3_E_INVALID, "t_by_mode[%d] is not finite", m);
    int j = 0;
    while (j < ms->n_t && ms->t[j] != t) ++j;
    if (j == ms->n_t) ms->t[ms->n_t++] = t;
    ms->t_index[m] = j;
  }
  if (target) {
    ms->has_target = 1;
    ms->t[ms->n_t] = t_target;
  }
  wd->w1 = w->w1;
  wd->w2 = w->w2;
  wd->w1_tgt = w->w1_tgt;
  wd->w2_tgt = w->w2_tgt;
  for (int m = 0; m < 3; ++m) wd->w_mod[m] = w->w_mod[m];
  wd->w_final = nullptr;
  return FLUX3_OK;
}

// Weight checks of a stack's blocks for the segments in use.
flux3_status check_stack_weights(const flux3_dims* d, const flux3_block_weights* per_mode,
                                 int32_t n_pm, const flux3_block_weights* joint,
                                 int32_t n_joint, const flux3_segment* segs, int32_t n_segs) {
  flux3_status r;
  if (n_pm > 0) {
    if (!per_mode) return fail(FLUX3_E_INVALID, "per_mode is NULL");
    for (int s = 0; s < n_segs; ++s)
      for (int b = 0; b < n_pm; ++b)
        if ((r = check_weights(&per_mode[segs[s].mode * n_pm + b], "per_mode",
                               segs[s].mode * n_pm + b, d)) != FLUX3_OK)
          return r;
  }
  if (n_joint > 0) {
    if (!joint) return fail(FLUX3_E_INVALID, "joint is NULL");
    for (int b = 0; b < n_joint; ++b)
      if ((r = check_weights(&joint[b], "joint", b, d)) != FLUX3_OK) return r;
  }
  return FLUX3_OK;
}

int64_t pad256(int64_t v) { return (v + 255) / 256 * 256; }

// Enqueues the two stages on validated arguments.
flux3_status run_stack(const flux3_dims* dims, const flux3_block_weights* per_mode, int32_t n_pm,
                       const flux3_block_weights* joint, int32_t n_joint, float* x,
                       int64_t n_tokens, const flux3_segment* segs, int32_t n_segs,
                       const flux3::SegTableHost& st, const float* mod_stage1,
                       const float* mod_stage2, int64_t mod_block_stride, const float* rope,
                       void* workspace, hipStream_t s) {
  flux3_status r;
  const size_t D = (size_t)dims->width;
  // stage 1: each segment runs its own mode's blocks on its rows alone.
  // Several segments go through one launch sequence per block when their
  // rows, each segment padded to 256, fit the workspace and their weights
  // share a layout: every segment is a row group with its mode's weight set
  // and attends within itself, so the result is that of separate blocks.
  if (n_pm > 0 && n_segs > 1) {
    flux3::RowGroups rg;
    memset(&rg, 0, sizeof rg);
    rg.n = n_segs;
    int64_t rows = 0;
    bool used[flux3::kMaxWeightSets] = {false, false, false};
    for (int sg = 0; sg < n_segs; ++sg) {
      used[segs[sg].mode] = true;
      rg.ws_start[sg] = (int32_t)rows;
      rg.x_start[sg] = segs[sg].start;
      rg.count[sg] = segs[sg].count;
      rg.wsel[sg] = segs[sg].mode;
      rows += pad256(segs[sg].count);
    }
    flux3_workspace_layout L;
    layout_of(dims, n_tokens, &L);
    bool grouped = rows <= L.n_pad;
    for (int b = 0; b < n_pm && grouped; ++b) {
      const flux3_block_weights& w0 = per_mode[segs[0].mode * n_pm + b];
      for (int sg = 1; sg < n_segs; ++sg)
        if (per_mode[segs[sg].mode * n_pm + b].layout != w0.layout) grouped = false;
    }
    if (grouped) {
      for (int b = 0; b < n_pm; ++b) {
        // set m holds mode m's block b; a mode no segment uses points at a
        // used mode's weights (never read, and never validated)
        flux3::WeightSets sets;
        sets.n = flux3::kMaxWeightSets;
        for (int m = 0; m < flux3::kMaxWeightSets; ++m)
          sets.w[m] = dev_weights(per_mode[(used[m] ? m : segs[0].mode) * n_pm + b]);
        r = run_block_groups(dims, sets, rg, rows, x, n_tokens, st,
                             mod_stage1 + (size_t)b * mod_block_stride, rope, workspace, n_tokens,
                             s, true);
        if (r != FLUX3_OK) return r;
      }
      n_pm = 0;
    }
  }
  for (int sg = 0; sg < n_segs && n_pm > 0; ++sg) {
    flux3::SegTableHost one;
    memset(&one, 0, sizeof one);
    one.n = 1;
    const int64_t start = segs[sg].start, cnt = segs[sg].count;
    for (int b = 0; b < n_pm; ++b) {
      const float* m1 = mod_stage1 + (size_t)b * mod_block_stride + (size_t)sg * 3 * D;
      r = run_block(dims, per_mode[segs[sg].mode * n_pm + b], x + start * D, cnt, one, m1,
                    rope + start * 128, workspace, s);
      if (r != FLUX3_OK) return r;
    }
  }
  // stage 2: joint blocks over the whole sequence
  for (int b = 0; b < n_joint; ++b) {
    r = run_block(dims, joint[b], x, n_tokens, st, mod_stage2 + (size_t)b * mod_block_stride,
                  rope, workspace, s);
    if (r != FLUX3_OK) return r;
  }
  return FLUX3_OK;
}

// Byte layout of flux3_transformer_forward's workspace.
struct TransformerLayout {
  size_t block, x, stage, w_out, mod1, mod2, mod_final, mod_ws, total;
  int64_t text_pad, img_pad, ref_pad;
};

void transformer_layout(const flux3_dims* d, const flux3_io_dims* io, int64_t n, int n_segs,
                        int64_t n_text, int64_t n_img, int64_t n_ref, TransformerLayout* L) {
  const size_t D = (size_t)d->width;
  L->text_pad = pad256(n_text);
  L->img_pad = pad256(n_img);
  L->ref_pad = pad256(n_ref);
  size_t off = 0;
  L->block = off;
  flux3_workspace_layout wl;
  layout_of(d, n, &wl);
  off = align_up(wl.total, kBufAlign);
  L->x = off;
  off = align_up(off + (size_t)n * D * 4, kBufAlign);
  L->stage = off;
  size_t stage = std::max((size_t)L->text_pad * io->text_dim,
                          (size_t)std::max(L->img_pad, L->ref_pad) * io->latent_dim) * 2;
  off = align_up(off + stage, kBufAlign);
  L->w_out = off;
  off = align_up(off + 256 * D * 2, kBufAlign);
  L->mod1 = off;
  off = align_up(off + (size_t)n_segs * 3 * D * 4, kBufAlign);
  L->mod2 = off;
  off = align_up(off + (size_t)n_segs * 3 * D * 4, kBufAlign);
  L->mod_final = off;
  off = align_up(off + 3 * D * 4, kBufAlign);
  L->mod_ws = off;
  off = align_up(off + flux3::modulation_workspace_floats((int)D) * 4, kBufAlign);
  L->total = off;
}

// Pieces per tile for a split linear: enough workgroups to cover the CUs,
// at least 4 k slices per piece, partials within the block workspace's
// split-partial region.
int split_pieces(int64_t m_pad, int64_t n_pad, int K) {
  const int64_t tiles = (m_pad / 256) * (n_pad / 256);
  const int nk = K / 64;
  int S = (int)std::max<int64_t>(1, (256 + tiles - 1) / tiles);
  S = std::min(S, std::max(1, nk / 4));
  const size_t budget = 2 * (size_t)flux3::kMaxSplitGroups * flux3::kSplitSlotBytes;
  while (S > 1 && (size_t)S * m_pad * n_pad * 4 > budget) --S;
  return S;
}

// One input or output linear through the split GEMM.
flux3_status io_linear(const void* a_packed, const void* w, bool w_packed, int64_t M,
                       int64_t m_pad, int N, int n_pad, int K, float* out, int ldo, float* part,
                       hipStream_t s) {
  flux3::SplitGemm g;
  g.a = a_packed;
  g.w = w;
  g.w_packed = w_packed;
  g.part = part;
  g.out = out;
  g.M = (int)M;
  g.m_pad = (int)m_pad;
  g.N = N;
  g.n_pad = n_pad;
  g.K = K;
  g.S = split_pieces(m_pad, n_pad, K);
  g.ldo = ldo;
  const int pi = prof_begin(FLUX3_K_IO_LINEARS, (double)M, s);
  hipError_t e = flux3::launch_gemm_split(g, s);
  prof_end(pi, s);
  return after_launch(e, "io_linear", s);
}

}  // namespace

// Entry points defined in other source files share these (abi_internal.hpp).
namespace flux3 {

flux3_status validate_block(const flux3_dims* dims, const flux3_block_weights* w, const float* x,
                            int64_t n_tokens, const flux3_segment* segs, int32_t n_segs,
                            const float* mod, const float* rope, SegTableHost* st) {
  flux3_status r = check_dims(dims);
  if (r != FLUX3_OK) return r;
  if (n_tokens < 0 || n_tokens > kMaxTokens)
    return fail(FLUX3_E_SHAPE, "n_tokens %lld outside [0, %lld]", (long long)n_tokens, (long long)kMaxTokens);
  if (n_tokens == 0) {
    if (n_segs != 0) return fail(FLUX3_E_SHAPE, "n_tokens is 0 but n_segs is %d", n_segs);
    return ok();
  }
  if ((r = check_weights(w, "w", 0, dims)) != FLUX3_OK) return r;
  if (!x || !mod || !rope) return fail(FLUX3_E_INVALID, "x, mod or rope is NULL");
  if (!aligned16(x) || !aligned16(mod) || !aligned16(rope))
    return fail(FLUX3_E_ALIGN, "x, mod or rope is not 16-byte aligned");
  return check_segments(segs, n_segs, n_tokens, st);
}

size_t block_buffer_bytes(const flux3_dims* dims, int64_t n_tokens) {
  flux3_workspace_layout L;
  layout_of(dims, n_tokens, &L);
  return L.part;
}

flux3_status run_block_whole_tiles(const flux3_dims* dims, const flux3_block_weights* w, float* x,
                                   int64_t n_tokens, const SegTableHost& st, const float* mod,
                                   const float* rope, void* buffers, void* stream) {
  flux3_status r = run_block(dims, *w, x, n_tokens, st, mod, rope, buffers,
                             static_cast<hipStream_t>(stream), /*split=*/false);
  return r == FLUX3_OK ? ok() : r;
}

flux3_status set_error(flux3_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof g_detail, fmt, ap);
  va_end(ap);
  return s;
}

}  // namespace flux3

extern "C" {

int64_t flux3_layout_tokens(const flux3_rope_layout* L) {
  if (!L) return -1;
  if (L->n_text < 0 || L->grid_h < 0 || L->grid_w < 0 || L->n_refs < 0 ||
      L->n_refs > FLUX3_MAX_REFS)
    return -1;
  if ((L->grid_h == 0) != (L->grid_w == 0)) return -1;
  int64_t n = (int64_t)L->n_text + (int64_t)L->grid_h * L->grid_w;
  if (L->n_refs > 0 && (!L->ref_h || !L->ref_w)) return -1;
  for (int k = 0; k < L->n_refs; ++k) {
    if (L->ref_h[k] <= 0 || L->ref_w[k] <= 0) return -1;
    n += (int64_t)L->ref_h[k] * L->ref_w[k];
  }
  return n;
}

flux3_status flux3_rope_tables_build(const flux3_rope_layout* layout, float* rope,
                                     int64_t n_tokens, void* stream) {
  if (!layout) return fail(FLUX3_E_INVALID, "layout is NULL");
  const int64_t n = flux3_layout_tokens(layout);
  if (n < 0) return fail(FLUX3_E_SHAPE, "invalid layout (negative size, n_refs > %d or missing ref arrays)", FLUX3_MAX_REFS);
  if (n != n_tokens)
    return fail(FLUX3_E_SHAPE, "layout has %lld tokens, n_tokens is %lld", (long long)n,
                (long long)n_tokens);
  if (n > kMaxTokens) return fail(FLUX3_E_SHAPE, "n_tokens %lld above %lld", (long long)n, (long long)kMaxTokens);
  if (n == 0) return ok();
  if (!rope) return fail(FLUX3_E_INVALID, "rope is NULL");
  if (!aligned16(rope)) return fail(FLUX3_E_ALIGN, "rope is not 16-byte aligned");
  flux3::RopeLayoutDev dl;
  memset(&dl, 0, sizeof dl);
  dl.n_text = layout->n_text;
  dl.grid_h = layout->grid_h;
  dl.grid_w = layout->grid_w;
  dl.n_refs = layout->n_refs;
  for (int k = 0; k < layout->n_refs; ++k) {
    dl.ref_h[k] = layout->ref_h[k];
    dl.ref_w[k] = layout->ref_w[k];
  }
  dl.theta = layout->theta;
  dl.hw_scale = layout->hw_scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int pi = prof_begin(FLUX3_K_ROPE_TABLES, (double)n, s);
  const hipError_t e = flux3::launch_rope_tables(dl, rope, n, s);
  prof_end(pi, s);
  flux3_status r = after_launch(e, "rope_tables", s);
  return r == FLUX3_OK ? ok() : r;
}

size_t flux3_workspace_bytes(const flux3_dims* dims, int64_t n_tokens) {
  if (check_dims(dims) != FLUX3_OK || n_tokens < 0 || n_tokens > kMaxTokens) return 0;
  flux3_workspace_layout L;
  layout_of(dims, n_tokens, &L);
  return L.total;
}

flux3_status flux3_workspace_layout_get(const flux3_dims* dims, int64_t n_tokens,
                                        flux3_workspace_layout* out) {
  flux3_status r = check_dims(dims);
  if (r != FLUX3_OK) return r;
  if (!out) return fail(FLUX3_E_INVALID, "out is NULL");
  if (n_tokens < 0 || n_tokens > kMaxTokens)
    return fail(FLUX3_E_SHAPE, "n_tokens %lld outside [0, %lld]", (long long)n_tokens, (long long)kMaxTokens);
  layout_of(dims, n_tokens, out);
  return ok();
}

size_t flux3_weights_packed_bytes(const flux3_dims* dims) {
  if (check_dims(dims) != FLUX3_OK) return 0;
  const size_t D = (size_t)dims->width, F = (size_t)dims->mlp_hidden;
  return 4 * align_up(D * D * 2, kBufAlign) + 3 * align_up(D * F * 2, kBufAlign);
}

flux3_status flux3_weights_pack(const flux3_dims* dims, const flux3_block_weights* in,
                                void* buffer, size_t buffer_bytes, flux3_block_weights* out,
                                void* stream) {
  flux3_status r = check_dims(dims);
  if (r != FLUX3_OK) return r;
  if ((r = check_weights(in, "in", 0, dims)) != FLUX3_OK) return r;
  if (in->layout != FLUX3_WEIGHTS_LINEAR)
    return fail(FLUX3_E_INVALID, "in is already packed");
  if (!out) return fail(FLUX3_E_INVALID, "out is NULL");
  if (!buffer) return fail(FLUX3_E_WORKSPACE, "buffer is NULL");
  if ((reinterpret_cast<uintptr_t>(buffer) & (kBufAlign - 1)) != 0)
    return fail(FLUX3_E_ALIGN, "buffer is not %zu-byte aligned", kBufAlign);
  const size_t need = flux3_weights_packed_bytes(dims);
  if (buffer_bytes < need)
    return fail(FLUX3_E_WORKSPACE, "buffer has %zu bytes, needs %zu", buffer_bytes, need);
  const int D = dims->width, F = dims->mlp_hidden;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const void* src[7] = {in->wq, in->wk, in->wv, in->wo, in->w_gate, in->w_up, in->w_down};
  const int rows[7] = {D, D, D, D, F, F, D};
  const int cols[7] = {D, D, D, D, D, D, F};
  static const char* names[7] = {"wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"};
  void* dst[7];
  char* b = static_cast<char*>(buffer);
  for (int i = 0; i < 7; ++i) {
    dst[i] = b;
    b += align_up((size_t)rows[i] * cols[i] * 2, kBufAlign);
    hipError_t e = flux3::launch_pack_rows(src[i], dst[i], rows[i], cols[i], s);
    if ((r = after_launch(e, names[i], s)) != FLUX3_OK) return r;
  }
  *out = *in;
  out->wq = dst[0]; out->wk = dst[1]; out->wv = dst[2]; out->wo = dst[3];
  out->w_gate = dst[4]; out->w_up = dst[5]; out->w_down = dst[6];
  out->layout = FLUX3_WEIGHTS_PACKED;
  return ok();
}

size_t flux3_weights_fp8r_bytes(const flux3_dims* dims) {
  if (check_dims(dims) != FLUX3_OK) return 0;
  const size_t D = (size_t)dims->width, F = (size_t)dims->mlp_hidden;
  return 4 * align_up(D * D, kBufAlign) + 3 * align_up(D * F, kBufAlign) +
         align_up((3 * D + 2 * F) * 4, kBufAlign) + align_up(D * 4, kBufAlign);
}

flux3_status flux3_weights_quantize_fp8r(const flux3_dims* dims, const flux3_block_weights* in,
                                         void* buffer, size_t buffer_bytes,
                                         flux3_block_weights* out, void* stream) {
  flux3_status r = check_dims(dims);
  if (r != FLUX3_OK) return r;
  if ((r = check_fp8_dims(dims)) != FLUX3_OK) return r;
  if ((r = check_weights(in, "in", 0, dims)) != FLUX3_OK) return r;
  if (in->layout != FLUX3_WEIGHTS_LINEAR)
    return fail(FLUX3_E_INVALID, "in must be in Linear layout");
  if (!out) return fail(FLUX3_E_INVALID, "out is NULL");
  if (!buffer) return fail(FLUX3_E_WORKSPACE, "buffer is NULL");
  if ((reinterpret_cast<uintptr_t>(buffer) & (kBufAlign - 1)) != 0)
    return fail(FLUX3_E_ALIGN, "buffer is not %zu-byte aligned", kBufAlign);
  const size_t need = flux3_weights_fp8r_bytes(dims);
  if (buffer_bytes < need)
    return fail(FLUX3_E_WORKSPACE, "buffer has %zu bytes, needs %zu", buffer_bytes, need);
  const int D = dims->width, F = dims->mlp_hidden;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // code matrices wq wk wv wo w_gate w_up w_down, then s_proj and s_out
  const size_t bytes[7] = {(size_t)D * D, (size_t)D * D, (size_t)D * D, (size_t)D * D,
                           (size_t)F * D, (size_t)F * D, (size_t)D * F};
  void* dst[7];
  char* b = static_cast<char*>(buffer);
  for (int i = 0; i < 7; ++i) {
    dst[i] = b;
    b += align_up(bytes[i], kBufAlign);
  }
  float* s_proj = reinterpret_cast<float*>(b);
  b += align_up((size_t)(3 * D + 2 * F) * 4, kBufAlign);
  float* s_out = reinterpret_cast<float*>(b);
  // the rows of [wq; wk; wv; w_gate; w_up], one matrix at a time
  struct Job {
    const void* w;
    void* out;
    int rows;
    size_t s_off;
    const char* name;
  };
  const Job jobs[5] = {{in->wq, dst[0], D, 0, "wq"},
                       {in->wk, dst[1], D, (size_t)D, "wk"},
                       {in->wv, dst[2], D, (size_t)2 * D, "wv"},
                       {in->w_gate, dst[4], F, (size_t)3 * D, "w_gate"},
                       {in->w_up, dst[5], F, (size_t)3 * D + F, "w_up"}};
  for (const Job& j : jobs) {
    hipError_t e = flux3::launch_quant_weight_rows(j.w, D, nullptr, 0, j.out, nullptr,
                                                   s_proj + j.s_off, j.rows, s);
    if ((r = after_launch(e, j.name, s)) != FLUX3_OK) return r;
  }
  // [wo | w_down]: one scale per output row over both matrices
  hipError_t e = flux3::launch_quant_weight_rows(in->wo, D, in->w_down, F, dst[3], dst[6], s_out,
                                                 D, s);
  if ((r = after_launch(e, "wo_w_down", s)) != FLUX3_OK) return r;
  *out = *in;
  out->wq = dst[0]; out->wk = dst[1]; out->wv = dst[2]; out->wo = dst[3];
  out->w_gate = dst[4]; out->w_up = dst[5]; out->w_down = dst[6];
  out->s_proj = s_proj;
  out->s_out = s_out;
  out->layout = FLUX3_WEIGHTS_FP8R;
  return ok();
}

flux3_status flux3_block_forward(const flux3_dims* dims, const flux3_block_weights* w, float* x,
                                 int64_t n_tokens, const flux3_segment* segs, int32_t n_segs,
                                 const float* mod, const float* rope, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  flux3::SegTableHost st;
  flux3_status r = flux3::validate_block(dims, w, x, n_tokens, segs, n_segs, mod, rope, &st);
  if (r != FLUX3_OK || n_tokens == 0) return r;
  flux3_workspace_layout L;
  if ((r = check_ws(dims, n_tokens, workspace, workspace_bytes, &L)) != FLUX3_OK) return r;
  r = run_block(dims, *w, x, n_tokens, st, mod, rope, workspace, static_cast<hipStream_t>(stream));
  return r == FLUX3_OK ? ok() : r;
}

flux3_status flux3_stack_forward(const flux3_dims* dims, const flux3_block_weights* per_mode,
                                 int32_t n_pm, const flux3_block_weights* joint, int32_t n_joint,
                                 float* x, int64_t n_tokens, const flux3_segment* segs,
                                 int32_t n_segs, const float* mod_stage1, const float* mod_stage2,
                                 int64_t mod_block_stride, const float* rope, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  flux3_status r = check_dims(dims);
  if (r != FLUX3_OK) return r;
  if (n_tokens < 0 || n_tokens > kMaxTokens)
    return fail(FLUX3_E_SHAPE, "n_tokens %lld outside [0, %lld]", (long long)n_tokens, (long long)kMaxTokens);
  if (n_pm < 0 || n_joint < 0) return fail(FLUX3_E_SHAPE, "n_pm %d / n_joint %d negative", n_pm, n_joint);
  if (mod_block_stride < 0) return fail(FLUX3_E_SHAPE, "mod_block_stride is negative");
  if (n_tokens == 0) {
    if (n_segs != 0) return fail(FLUX3_E_SHAPE, "n_tokens is 0 but n_segs is %d", n_segs);
    return ok();
  }
  if (!x || !rope) return fail(FLUX3_E_INVALID, "x or rope is NULL");
  if (!aligned16(x) || !aligned16(rope)) return fail(FLUX3_E_ALIGN, "x or rope is not 16-byte aligned");
  flux3::SegTableHost st;
  if ((r = check_segments(segs, n_segs, n_tokens, &st)) != FLUX3_OK) return r;
  if (n_pm > 0) {
    if (!mod_stage1) return fail(FLUX3_E_INVALID, "mod_stage1 is NULL");
    if (!aligned16(mod_stage1)) return fail(FLUX3_E_ALIGN, "mod_stage1 is not 16-byte aligned");
  }
  if (n_joint > 0) {
    if (!mod_stage2) return fail(FLUX3_E_INVALID, "mod_stage2 is NULL");
    if (!aligned16(mod_stage2)) return fail(FLUX3_E_ALIGN, "mod_stage2 is not 16-byte aligned");
  }
  if ((r = check_stack_weights(dims, per_mode, n_pm, joint, n_joint, segs, n_segs)) != FLUX3_OK)
    return r;
  if (mod_block_stride % 4 != 0)
    return fail(FLUX3_E_ALIGN, "mod_block_stride must be a multiple of 4 floats");
  flux3_workspace_layout L;
  if ((r = check_ws(dims, n_tokens, workspace, workspace_bytes, &L)) != FLUX3_OK) return r;
  if ((r = run_stack(dims, per_mode, n_pm, joint, n_joint, x, n_tokens, segs, n_segs, st,
                     mod_stage1, mod_stage2, mod_block_stride, rope, workspace,
                     static_cast<hipStream_t>(stream))) != FLUX3_OK)
    return r;
  return ok();
}

size_t flux3_modulation_workspace_bytes(const flux3_dims* dims) {
  if (check_dims(dims) != FLUX3_OK) return 0;
  return align_up(flux3::modulation_workspace_floats(dims->width) * sizeof(float), kBufAlign);
}



flux3_status flux3_modulation_forward(const flux3_dims* dims, const flux3_modulation_weights* w,
                                      const float* t_by_mode, float t_target,
                                      const flux3_segment* segs, int32_t n_segs, float* mod,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  flux3_status r = check_dims(dims);
  if (r != FLUX3_OK) return r;
  if (!segs || n_segs < 1) return fail(FLUX3_E_SHAPE, "n_segs %d (need >= 1) or segs NULL", n_segs);
  if (n_segs > FLUX3_MAX_SEGMENTS) return fail(FLUX3_E_SHAPE, "n_segs %d > %d", n_segs, FLUX3_MAX_SEGMENTS);
  const int64_t n = (int64_t)segs[n_segs - 1].start + segs[n_segs - 1].count;
  if (n < 1 || n > kMaxTokens) return fail(FLUX3_E_SHAPE, "segments cover %lld tokens", (long long)n);
  flux3::SegTableHost st;
  if ((r = check_segments(segs, n_segs, n, &st)) != FLUX3_OK) return r;
  flux3::ModulationShape ms;
  flux3::ModulationWeightsDev wd;
  int32_t seg_mode[FLUX3_MAX_SEGMENTS];
  if ((r = prepare_modulation(dims, w, t_by_mode, t_target, segs, n_segs, &ms, &wd, seg_mode)) !=
      FLUX3_OK)
    return r;
  if (!mod) return fail(FLUX3_E_INVALID, "mod is NULL");
  if (!aligned16(mod)) return fail(FLUX3_E_ALIGN, "mod is not 16-byte aligned");
  const size_t need = flux3_modulation_workspace_bytes(dims);
  if (!workspace) return fail(FLUX3_E_INVALID, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & (kBufAlign - 1)) != 0)
    return fail(FLUX3_E_ALIGN, "workspace is not %zu-byte aligned", kBufAlign);
  if (workspace_bytes < need)
    return fail(FLUX3_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int pi = prof_begin(FLUX3_K_MODULATION, (double)n, s);
  hipError_t e = flux3::launch_modulation(ms, wd, st, seg_mode, mod, static_cast<float*>(workspace), s);
  prof_end(pi, s);
  if ((r = after_launch(e, "modulation", s)) != FLUX3_OK) return r;
  return ok();
}

size_t flux3_transformer_workspace_bytes(const flux3_dims* dims, const flux3_io_dims* io_dims,
                                         int64_t n_tokens) {
  if (check_dims(dims) != FLUX3_OK || !io_dims || io_dims->text_dim <= 0 ||
      io_dims->text_dim % 64 != 0 || io_dims->text_dim > kMaxTextDim || io_dims->latent_dim <= 0 || io_dims->latent_dim % 64 != 0 ||
      io_dims->latent_dim > 256 || n_tokens < 0 || n_tokens > kMaxTokens)
    return 0;
  TransformerLayout L;
  // sized for the worst split of n_tokens between text, image and references
  transformer_layout(dims, io_dims, n_tokens, FLUX3_MAX_SEGMENTS, n_tokens, n_tokens, n_tokens, &L);
  return L.total;
}

flux3_status flux3_transformer_forward(const flux3_dims* dims, const flux3_io_dims* io_dims,
                                       const flux3_io_weights* io,
                                       const flux3_modulation_weights* mod_w,
                                       const flux3_block_weights* per_mode, int32_t n_pm,
                                       const flux3_block_weights* joint, int32_t n_joint,
                                       const void* text, const float* image, const float* refs,
                                       const flux3_segment* segs, int32_t n_segs, float t,
                                       float t_target, const float* rope, float* velocity,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  flux3_status r = check_dims(dims);
  if (r != FLUX3_OK) return r;
  if (!io_dims) return fail(FLUX3_E_INVALID, "io_dims is NULL");
  const int TD = io_dims->text_dim, LD = io_dims->latent_dim;
  if (TD <= 0 || TD % 64 != 0 || TD > kMaxTextDim)
    return fail(FLUX3_E_UNSUPPORTED, "text_dim %d unsupported (positive multiple of 64, at most %d)",
                TD, kMaxTextDim);
  if (LD <= 0 || LD % 64 != 0 || LD > 256)
    return fail(FLUX3_E_UNSUPPORTED, "latent_dim %d unsupported (multiple of 64, <= 256)", LD);
  if (!io) return fail(FLUX3_E_INVALID, "io weights struct is NULL");
  if (!mod_w) return fail(FLUX3_E_INVALID, "mod_w is NULL");
  if (n_pm < 0 || n_joint < 0) return fail(FLUX3_E_SHAPE, "n_pm %d / n_joint %d negative", n_pm, n_joint);
  if (!segs || n_segs < 1 || n_segs > FLUX3_MAX_SEGMENTS)
    return fail(FLUX3_E_SHAPE, "n_segs %d outside [1, %d] or segs NULL", n_segs, FLUX3_MAX_SEGMENTS);
  const int64_t n = (int64_t)segs[n_segs - 1].start + segs[n_segs - 1].count;
  if (n < 1 || n > kMaxTokens) return fail(FLUX3_E_SHAPE, "segments cover %lld tokens", (long long)n);
  flux3::SegTableHost st;
  if ((r = check_segments(segs, n_segs, n, &st)) != FLUX3_OK) return r;
  int64_t n_text = 0, n_img = 0, n_ref = 0;
  int img_seg = -1, text_segs = 0;
  for (int i = 0; i < n_segs; ++i) {
    if (segs[i].mode == FLUX3_MODE_TEXT) { n_text += segs[i].count; ++text_segs; }
    if (segs[i].mode == FLUX3_MODE_IMAGE) {
      if (img_seg >= 0) return fail(FLUX3_E_SHAPE, "more than one image segment");
      img_seg = i;
      n_img = segs[i].count;
    }
    if (segs[i].mode == FLUX3_MODE_REF) n_ref += segs[i].count;
  }
  if (img_seg < 0) return fail(FLUX3_E_SHAPE, "no image segment");
  if (text_segs > 1) return fail(FLUX3_E_SHAPE, "more than one text segment");
  // weights and inputs
  struct { const void* p; const char* name; bool need; } req[] = {
      {io->w_text, "w_text", n_text > 0}, {io->w_img_in, "w_img_in", true},
      {io->w_ref_in, "w_ref_in", n_ref > 0}, {io->w_final, "w_final", true},
      {io->w_out, "w_out", true},         {text, "text", n_text > 0},
      {image, "image", true},             {refs, "refs", n_ref > 0},
      {rope, "rope", true},               {velocity, "velocity", true}};
  for (const auto& q : req) {
    if (!q.need) continue;
    if (!q.p) return fail(FLUX3_E_INVALID, "%s is NULL", q.name);
    if (!aligned16(q.p)) return fail(FLUX3_E_ALIGN, "%s is not 16-byte aligned", q.name);
  }
  if (!std::isfinite(t)) return fail(FLUX3_E_INVALID, "t is not finite");
  if ((r = check_stack_weights(dims, per_mode, n_pm, joint, n_joint, segs, n_segs)) != FLUX3_OK)
    return r;
  flux3::ModulationShape ms[2];
  flux3::ModulationWeightsDev wd[2];
  int32_t seg_mode[FLUX3_MAX_SEGMENTS];
  const float t_by_mode[3] = {0.f, t, 0.f};
  for (int k = 0; k < 2; ++k)
    if ((r = prepare_modulation(dims, &mod_w[k], t_by_mode, t_target, segs, n_segs, &ms[k], &wd[k],
                                seg_mode)) != FLUX3_OK)
      return r;
  wd[1].w_final = io->w_final;
  TransformerLayout L;
  transformer_layout(dims, io_dims, n, n_segs, n_text, n_img, n_ref, &L);
  if (!workspace) return fail(FLUX3_E_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & (kBufAlign - 1)) != 0)
    return fail(FLUX3_E_ALIGN, "workspace is not %zu-byte aligned", kBufAlign);
  if (workspace_bytes < L.total)
    return fail(FLUX3_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  flux3_workspace_layout bl;
  layout_of(dims, n, &bl);
  const flux3::WsPtrs wp = carve(base + L.block, bl);
  float* part = static_cast<float*>(wp.part);
  float* x = reinterpret_cast<float*>(base + L.x);
  void* stage = base + L.stage;
  const int D = dims->width;
  hipError_t e;
  // input projections into the residual stream, in sequence order
  const int64_t img0 = segs[img_seg].start;
  struct { const void* in; bool f32; int64_t rows, pad, row0; int K; const void* w; } inp[3] = {
      {text, false, n_text, L.text_pad, 0, TD, io->w_text},
      {image, true, n_img, L.img_pad, img0, LD, io->w_img_in},
      {refs, true, n_ref, L.ref_pad, img0 + n_img, LD, io->w_ref_in}};
  for (const auto& q : inp) {
    if (q.rows == 0) continue;
    e = flux3::launch_pack_input(q.in, q.f32, stage, (int)q.rows, (int)q.pad, q.K, s);
    if ((r = after_launch(e, "pack_input", s)) != FLUX3_OK) return r;
    if ((r = io_linear(stage, q.w, false, q.rows, q.pad, D, D, q.K, x + q.row0 * D, D, part, s)) !=
        FLUX3_OK)
      return r;
  }
  // both stages' modulation; stage 2 also gives the output layer's
  float* mod1 = reinterpret_cast<float*>(base + L.mod1);
  float* mod2 = reinterpret_cast<float*>(base + L.mod2);
  float* modf = reinterpret_cast<float*>(base + L.mod_final);
  float* mws = reinterpret_cast<float*>(base + L.mod_ws);
  for (int k = 0; k < 2; ++k) {
    const int pi = prof_begin(FLUX3_K_MODULATION, (double)n, s);
    e = flux3::launch_modulation(ms[k], wd[k], st, seg_mode, k ? mod2 : mod1, mws, s,
                                 k ? modf : nullptr);
    prof_end(pi, s);
    if ((r = after_launch(e, "modulation", s)) != FLUX3_OK) return r;
  }
  if ((r = run_stack(dims, per_mode, n_pm, joint, n_joint, x, n, segs, n_segs, st, mod1, mod2, 0,
                     rope, base + L.block, s)) != FLUX3_OK)
    return r;
  // output layer on the image rows: modulated LayerNorm into h, then W_out
  flux3::BlockShape bs;
  bs.M = (int32_t)n_img;
  bs.n_pad = (int32_t)L.img_pad;
  bs.D = D;
  bs.H = dims->heads;
  bs.F = dims->mlp_hidden;
  bs.rows = (int32_t)L.img_pad;
  bs.rg = flux3::one_group((int32_t)n_img);
  flux3::SegTableHost one;
  memset(&one, 0, sizeof one);
  one.n = 1;
  int pi = prof_begin(FLUX3_K_LN_MODULATE, (double)n_img, s);
  e = flux3::launch_ln_modulate(bs, x + img0 * D, modf, one, wp.h, kEpsLN, s);
  prof_end(pi, s);
  if ((r = after_launch(e, "ln_modulate", s)) != FLUX3_OK) return r;
  void* w_out = base + L.w_out;   // W_out packed, zero rows up to 256
  e = flux3::launch_pack_input(io->w_out, false, w_out, LD, 256, D, s);
  if ((r = after_launch(e, "pack_input", s)) != FLUX3_OK) return r;
  if ((r = io_linear(wp.h, w_out, true, n_img, L.img_pad, LD, 256, D, velocity, LD, part, s)) !=
      FLUX3_OK)
    return r;
  return ok();
}

flux3_status flux3_sigmas(int32_t steps, double shift, float* sigmas) {
  if (steps < 1) return fail(FLUX3_E_SHAPE, "steps %d < 1", steps);
  if (!sigmas) return fail(FLUX3_E_INVALID, "sigmas is NULL");
  if (!(shift > 0.0) || !std::isfinite(shift)) return fail(FLUX3_E_INVALID, "shift must be positive");
  for (int i = 0; i < steps; ++i) {
    // evenly spaced from 1 down to 1/steps
    const double sg = steps == 1 ? 1.0 : 1.0 + i * ((1.0 / steps - 1.0) / (steps - 1));
    sigmas[i] = (float)(shift * sg / (1.0 + (shift - 1.0) * sg));
  }
  sigmas[steps] = 0.f;
  return ok();
}

flux3_status flux3_euler_step(const float* v, float* latent, float* x0_preview, int64_t n,
                              float sigma, float sigma_next, void* stream) {
  if (!v || !latent) return fail(FLUX3_E_INVALID, "v or latent is NULL");
  if (!aligned16(v) || !aligned16(latent) || (x0_preview && !aligned16(x0_preview)))
    return fail(FLUX3_E_ALIGN, "v, latent or x0_preview is not 16-byte aligned");
  if (n < 0 || n % 4 != 0) return fail(FLUX3_E_SHAPE, "n %lld must be a non-negative multiple of 4", (long long)n);
  if (!std::isfinite(sigma) || !std::isfinite(sigma_next))
    return fail(FLUX3_E_INVALID, "sigma or sigma_next is not finite");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int pi = prof_begin(FLUX3_K_EULER, (double)n, s);
  hipError_t e = flux3::launch_euler(v, latent, x0_preview, n, sigma, sigma_next, s);
  prof_end(pi, s);
  flux3_status r = after_launch(e, "euler", s);
  return r != FLUX3_OK ? r : ok();
}

size_t flux3_sample_workspace_bytes(const flux3_dims* dims, const flux3_io_dims* io_dims,
                                    int64_t n_tokens) {
  const size_t t = flux3_transformer_workspace_bytes(dims, io_dims, n_tokens);
  if (t == 0) return 0;
  return t + align_up((size_t)n_tokens * io_dims->latent_dim * 4, kBufAlign);
}

flux3_status flux3_sample(const flux3_dims* dims, const flux3_io_dims* io_dims,
                          const flux3_io_weights* io, const flux3_modulation_weights* mod_w,
                          const flux3_block_weights* per_mode, int32_t n_pm,
                          const flux3_block_weights* joint, int32_t n_joint, const void* text,
                          float* latent, const float* refs, const flux3_segment* segs,
                          int32_t n_segs, int32_t steps, double shift, int32_t distilled,
                          const float* rope, float* previews, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (steps < 1 || steps > 1000) return fail(FLUX3_E_SHAPE, "steps %d outside [1, 1000]", steps);
  std::vector<float> sig(steps + 1);
  flux3_status r = flux3_sigmas(steps, shift, sig.data());
  if (r != FLUX3_OK) return r;
  if (!dims || !io_dims) return fail(FLUX3_E_INVALID, "dims or io_dims is NULL");
  if (!segs || n_segs < 1 || n_segs > FLUX3_MAX_SEGMENTS)
    return fail(FLUX3_E_SHAPE, "n_segs %d outside [1, %d] or segs NULL", n_segs, FLUX3_MAX_SEGMENTS);
  const int64_t n = (int64_t)segs[n_segs - 1].start + segs[n_segs - 1].count;
  int64_t n_img = 0;
  for (int i = 0; i < n_segs; ++i)
    if (segs[i].mode == FLUX3_MODE_IMAGE) n_img += segs[i].count;
  if (previews && !aligned16(previews)) return fail(FLUX3_E_ALIGN, "previews is not 16-byte aligned");
  const size_t need = flux3_sample_workspace_bytes(dims, io_dims, n);
  if (need == 0) return fail(FLUX3_E_UNSUPPORTED, "dims or io_dims unsupported");
  if (!workspace) return fail(FLUX3_E_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(FLUX3_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  const size_t tbytes = flux3_transformer_workspace_bytes(dims, io_dims, n);
  float* vel = reinterpret_cast<float*>(static_cast<char*>(workspace) + tbytes);
  const int64_t nv = n_img * io_dims->latent_dim;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int i = 0; i < steps; ++i) {
    // the first call validates every argument before anything is enqueued
    r = flux3_transformer_forward(dims, io_dims, io, mod_w, per_mode, n_pm, joint, n_joint, text,
                                  latent, refs, segs, n_segs, sig[i],
                                  distilled ? sig[i + 1] : -1.f, rope, vel, workspace, tbytes,
                                  stream);
    if (r != FLUX3_OK) return r;
    const int pi = prof_begin(FLUX3_K_EULER, (double)nv, s);
    hipError_t e = flux3::launch_euler(vel, latent, previews ? previews + (size_t)i * nv : nullptr,
                                       nv, sig[i], sig[i + 1], s);
    prof_end(pi, s);
    if ((r = after_launch(e, "euler", s)) != FLUX3_OK) return r;
  }
  return ok();
}

flux3_status flux3_device_query(int32_t device, flux3_device_info* out) {
  if (!out) return fail(FLUX3_E_INVALID, "out is NULL");
  memset(out, 0, sizeof *out);
  int cus = 0, clk = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&clk, hipDeviceAttributeClockRate, device);
  hipDeviceProp_t prop;
  if (e == hipSuccess) e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return fail(FLUX3_E_HIP, "device %d query: %s", device, hipGetErrorString(e));
  out->compute_units = cus;
  out->clock_khz = clk;
  out->bf16_dense_tflops = (double)cus * (double)clk * 1e3 * 4096.0 / 1e12;
  snprintf(out->arch, sizeof out->arch, "%s", prop.gcnArchName);
  return ok();
}

void flux3_set_debug_sync(int32_t on) { g_debug_sync.store(on, std::memory_order_relaxed); }

void flux3_profile_enable(int32_t on) { g_prof_on = on != 0; }

void flux3_profile_reset(void) {
  for (const ProfRec& r : g_prof) {
    (void)hipEventSynchronize(r.b);
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
}

namespace {
// Stats of the records of one kind, those with token count m only when
// m >= 0.
flux3_status profile_stats(int32_t kernel, int64_t m, flux3_kernel_stats* out) {
  if (!out) return fail(FLUX3_E_INVALID, "out is NULL");
  if (kernel < 0 || kernel >= FLUX3_K_COUNT) return fail(FLUX3_E_INVALID, "kernel kind %d", kernel);
  flux3_kernel_stats st = {0, 0.0, 0.0, 0.0};
  for (const ProfRec& r : g_prof) {
    if (r.kind != kernel || (m >= 0 && r.m != (double)m)) continue;
    hipError_t e = hipEventSynchronize(r.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return fail(FLUX3_E_HIP, "event read: %s", hipGetErrorString(e));
    st.launches += 1;
    st.total_ms += ms;
    st.tokens += r.m;
    st.tokens_sq += r.m2;
  }
  *out = st;
  return ok();
}
}  // namespace

flux3_status flux3_profile_read(int32_t kernel, flux3_kernel_stats* out) {
  return profile_stats(kernel, -1, out);
}

flux3_status flux3_profile_read_tokens(int32_t kernel, int64_t n_tokens,
                                       flux3_kernel_stats* out) {
  if (n_tokens < 0) return fail(FLUX3_E_SHAPE, "n_tokens %lld is negative", (long long)n_tokens);
  return profile_stats(kernel, n_tokens, out);
}

const char* flux3_status_string(flux3_status s) {
  switch (s) {
    case FLUX3_OK: return "ok";
    case FLUX3_E_INVALID: return "invalid argument";
    case FLUX3_E_SHAPE: return "inconsistent shape or segments";
    case FLUX3_E_UNSUPPORTED: return "unsupported dims";
    case FLUX3_E_ALIGN: return "misaligned pointer";
    case FLUX3_E_WORKSPACE: return "workspace missing or too small";
    case FLUX3_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* flux3_last_error_detail(void) { return g_detail; }

}  // extern "C"
