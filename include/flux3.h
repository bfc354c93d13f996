/*
 * flux3.h -- C ABI of libflux3, the MI355X (gfx950) forward path of the
 * FLUX.3 Image Klein transformer block and its two-stage stack.
 *
 * Sources (release pages, cited by title and section):
 *   [P1] "FLUX.3 Image Klein Is Now Available in Diffusers" (15jq.com),
 *        section "Speed, architecture, and how the tokens move".
 *   [P3] Chinese translation of the Diffusers release post (everytik.com):
 *        the block listing (shift, scale and gate arguments) and the RoPE
 *        position table; the modular pipeline's `prepare_rope_inputs` step.
 *   [P4] "How to Run FLUX 3 Image Klein Locally" (rohitghumare.com),
 *        sections "Inside the transformer", "The latent space and the VAE".
 *   [P5] ifeeling.app summary, architecture paragraphs (reference tokens
 *        are offset negatively along l).
 *
 * Conventions shared by every entry point
 *   - Device pointers are caller-owned HIP device memory; the library never
 *     allocates, frees or keeps any of them past the call.  Host pointers
 *     (segment lists, weight-struct arrays, layout arrays, dims) are read
 *     during the call only.  The library allocates nothing and keeps
 *     nothing across calls, with two stated exceptions: the fixed per-GPU
 *     array of flux3_block_forward_noalloc, and the HIP events of the
 *     opt-in kernel timing (flux3_profile_*).
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream.  Calls only enqueue work and return; results are ready after
 *     the caller synchronises that stream.
 *   - All arguments are validated on the host before anything is enqueued;
 *     a non-zero status means nothing was enqueued.  After enqueue, a HIP
 *     launch error maps to FLUX3_E_HIP.  Device faults surface at the
 *     caller's next synchronisation.  No C++ exception crosses the ABI.
 *     flux3_last_error_detail() returns a per-thread message for the last
 *     failing call.
 *   - bf16 is bfloat16 (IEEE binary32 upper half); accumulation is fp32.
 *   - Device pointers must be 16-byte aligned (FLUX3_E_ALIGN otherwise).
 *   - Supported dims: head_dim == 128, heads a positive even number up
 *     to 512, width == heads * 128, mlp_hidden a positive multiple of 128
 *     up to 262144 (FLUX3_E_UNSUPPORTED otherwise); n_tokens at most 2^20.
 *     The model's are width 3072, 24 heads, 128, SwiGLU hidden 9216 [P4].
 */
#ifndef FLUX3_H
#define FLUX3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t flux3_status;
enum {
  FLUX3_OK = 0,
  FLUX3_E_INVALID = -1,     /* null pointer, bad mode or enum value          */
  FLUX3_E_SHAPE = -2,       /* sizes or segments inconsistent                */
  FLUX3_E_UNSUPPORTED = -3, /* dims outside what the kernels implement       */
  FLUX3_E_ALIGN = -4,       /* device pointer not 16-byte aligned            */
  FLUX3_E_WORKSPACE = -5,   /* workspace missing or smaller than required    */
  FLUX3_E_HIP = -6          /* HIP runtime reported an error                 */
};

#define FLUX3_MAX_SEGMENTS 16
#define FLUX3_MAX_REFS 15

/* Token modes, in the order the joint sequence concatenates them [P1]. */
enum { FLUX3_MODE_TEXT = 0, FLUX3_MODE_IMAGE = 1, FLUX3_MODE_REF = 2 };

typedef struct {
  int32_t width;      /* model width D (3072)                  */
  int32_t heads;      /* attention heads (24)                  */
  int32_t head_dim;   /* per-head dims, must be 128            */
  int32_t mlp_hidden; /* SwiGLU hidden width F (9216)          */
} flux3_dims;

/* A contiguous run of tokens of one kind.  Segments passed to a call must
 * tile [0, n_tokens) in order, each with count > 0, and with modes in the
 * sequence order text, image, reference (non-decreasing mode) [P1]. */
typedef struct {
  int32_t start;
  int32_t count;
  int32_t mode; /* FLUX3_MODE_* */
} flux3_segment;

/* Layouts of a block's weight matrices (flux3_block_weights.layout). */
enum { FLUX3_WEIGHTS_LINEAR = 0, FLUX3_WEIGHTS_PACKED = 1, FLUX3_WEIGHTS_FP8R = 2 };

/* One block's weights, all device pointers.  Matrices are bf16, no biases
 * [P3 block listing; P4], in torch Linear layout [out][in] row-major
 * (layout = FLUX3_WEIGHTS_LINEAR, the zero value) or in the packed operand
 * layout that flux3_weights_pack writes (FLUX3_WEIGHTS_PACKED), or rowwise
 * e4m3 codes that flux3_weights_quantize_fp8r writes (FLUX3_WEIGHTS_FP8R):
 *   wq, wk, wv, wo : [width][width]
 *   w_gate, w_up   : [mlp_hidden][width]   (silu acts on the w_gate branch)
 *   w_down         : [width][mlp_hidden]
 *   q_norm, k_norm : fp32 [head_dim] RMSNorm scales for queries and keys.
 *   s_proj, s_out  : FLUX3_WEIGHTS_FP8R only (ignored otherwise): fp32
 *                    dequantisation scale of each output row, s_proj
 *                    [3 width + 2 mlp_hidden] for the rows of wq, wk, wv,
 *                    w_gate, w_up in that order, s_out [width] for the rows
 *                    of the output linear [wo | w_down]. */
typedef struct {
  const void *wq, *wk, *wv, *wo;
  const void *w_gate, *w_up, *w_down;
  const float *q_norm, *k_norm;
  int32_t layout;
  const float *s_proj, *s_out;
} flux3_block_weights;

/* Bytes of one block's seven matrices in the packed operand layout (each
 * matrix starts on a 256-byte boundary); 0 if dims are unsupported. */
size_t flux3_weights_packed_bytes(const flux3_dims *dims);

/* Copies one block's Linear-layout matrices into buffer in the packed
 * operand layout the GEMMs load from (the same layout as the workspace's
 * packed activations, see flux3_workspace_layout_get): an [R][K] matrix
 * becomes 1-KiB blocks of 8 rows x 64 k, so that every direct load of the
 * GEMMs' weight slices moves one contiguous KiB instead of 8 row pieces of
 * 128 bytes.  Done once per weight set (weights are static); the block
 * results are bit-identical to those from the Linear layout.
 *   in     : layout FLUX3_WEIGHTS_LINEAR, all pointers valid and aligned.
 *   buffer : device, >= flux3_weights_packed_bytes(dims), 256-byte aligned;
 *            owned by the caller and must outlive every use of *out.
 *   out    : host struct filled with pointers into buffer, the norm
 *            pointers of in, and layout FLUX3_WEIGHTS_PACKED.
 * Asynchronous on stream.  Errors: FLUX3_E_INVALID (null or packed in),
 * FLUX3_E_UNSUPPORTED (dims), FLUX3_E_ALIGN, FLUX3_E_WORKSPACE (buffer too
 * small), FLUX3_E_HIP. */
flux3_status flux3_weights_pack(const flux3_dims *dims, const flux3_block_weights *in,
                                void *buffer, size_t buffer_bytes, flux3_block_weights *out,
                                void *stream);

/* Bytes of one block's weights in the rowwise-FP8 form: the seven code
 * matrices (one byte per value) and the two scale arrays, each on a
 * 256-byte boundary; 0 if dims are unsupported. */
size_t flux3_weights_fp8r_bytes(const flux3_dims *dims);

/* The rowwise-FP8 ("fp8r") form of one block's weights [P1 "Smaller GPUs,
 * single files, and custom LoRA training": the rowwise-FP8 single file;
 * P4 "What Black Forest Labs released": FP8 files and FP8 kernels].
 * Each output row of the block's two fused linears, [wq; wk; wv; w_gate;
 * w_up] (over width inputs) and [wo | w_down] (over width + mlp_hidden
 * inputs), with largest magnitude a gets the scale s = a / 448 and the
 * e4m3 codes (OCP 8-bit float: bias 7, 3 mantissa bits, largest 448) of
 * its values times 448 / a: nearest, ties to the even code, clamped to
 * +-448, every step in fp32; an all-zero row gets s = 0 and zero codes.
 * A block run with these weights quantises its two GEMM inputs, the
 * modulated h and [o | act], the same way per token row and runs both
 * GEMMs on the fp8 matrix cores with fp32 accumulation; the rest of the
 * block is unchanged.  Done once per weight set.
 *   in     : layout FLUX3_WEIGHTS_LINEAR, all pointers valid and aligned.
 *   buffer : device, >= flux3_weights_fp8r_bytes(dims), 256-byte aligned;
 *            owned by the caller and must outlive every use of *out.
 *   out    : host struct with the code matrices and scales in buffer, the
 *            norm pointers of in, and layout FLUX3_WEIGHTS_FP8R.  A code
 *            matrix [R][K] is stored in the packed fp8 layout: 1-KiB blocks
 *            of 8 rows x 128 codes, block (row / 8, k / 128) at block index
 *            (row / 8) (K / 128) + k / 128, row row % 8 taking 128 bytes of
 *            it, its 16-byte chunk c (codes 16c .. 16c + 15) in slot
 *            c ^ ((row / 2) % 8).
 * Asynchronous on stream.  Errors: FLUX3_E_INVALID (null or not Linear
 * in), FLUX3_E_UNSUPPORTED (dims; also width + mlp_hidden > 16384 or
 * mlp_hidden >= 7 width, where the per-token codes of [o | act] would not
 * fit the block workspace), FLUX3_E_ALIGN, FLUX3_E_WORKSPACE (buffer too
 * small), FLUX3_E_HIP. */
flux3_status flux3_weights_quantize_fp8r(const flux3_dims *dims, const flux3_block_weights *in,
                                         void *buffer, size_t buffer_bytes,
                                         flux3_block_weights *out, void *stream);

/* Token layout of one call: n_text text tokens, a grid_h x grid_w noisy
 * image grid (raster order), then n_refs reference grids ref_h[k] x ref_w[k]
 * (host arrays).  theta is the RoPE base (10000 in this build's reading);
 * hw_scale multiplies a grid row/col to give its h/w position (0.5 is the
 * row/2, col/2 of the page table). */
typedef struct {
  int32_t n_text, grid_h, grid_w, n_refs;
  const int32_t *ref_h, *ref_w;
  double theta;
  double hw_scale;
} flux3_rope_layout;

/* Number of tokens a layout describes; -1 if the layout is invalid. */
int64_t flux3_layout_tokens(const flux3_rope_layout *layout);

/* Rotary tables for a layout: the pipeline's prepare_rope_inputs step,
 * run once per layout outside the block loop [P3 modular pipeline].
 * Positions follow the page table [P3 RoPE table; P5]:
 *   text token i            -> (t, h, w, l) = (0, 0, 0, i)
 *   image token (row, col)  -> (0, row*hw_scale, col*hw_scale, 0)
 *   reference k (row, col)  -> (0, row*hw_scale, col*hw_scale, -(k+1))
 * Each 128-dim head gives every axis (t, h, w, l) 32 dims [P1]: pair
 * p = 16a + j rotates by angle pos[a] * theta^(-2j/32).
 * Output rope: device fp32 [n_tokens][64][2] = (cos, sin), computed in fp64
 * and rounded once to fp32.  n_tokens must equal flux3_layout_tokens().
 * Errors: FLUX3_E_INVALID (null), FLUX3_E_SHAPE (token count mismatch,
 * negative sizes, n_refs > FLUX3_MAX_REFS), FLUX3_E_ALIGN. */
flux3_status flux3_rope_tables_build(const flux3_rope_layout *layout,
                                     float *rope, int64_t n_tokens,
                                     void *stream);

/* Workspace bytes block_forward / stack_forward need for n_tokens tokens
 * (about 48 KiB per token at the model dims, plus a fixed 128 MiB of
 * split-tile partial sums); 0 if dims are unsupported. */
size_t flux3_workspace_bytes(const flux3_dims *dims, int64_t n_tokens);

/* Byte offsets of the intermediates a block leaves in the workspace, so a
 * caller can inspect them after the call: h = modulated LayerNorm output
 * bf16 [n_pad][width], packed (below); q, k = RMS-normalised, rotated
 * queries/keys bf16 [heads][n_pad][128]; vt = values bf16 [heads][128][n_pad]
 * with keys permuted inside every 16 (groups of 4 in the order 0, 2, 1, 3);
 * cat = bf16 [n_pad][width + mlp_hidden], packed, holding the attention
 * output in columns [0, width) and silu(gate)*up in [width, width +
 * mlp_hidden).  Packed: a [R][K] matrix is stored as 1-KiB blocks of 8 rows
 * x 64 columns, block (r/8, c/64) at block index (r/8)*(K/64) + c/64; in a
 * block, row r%8 takes 128 bytes whose 16-byte chunk j (columns 8j..8j+7 of
 * the block) sits at chunk position j ^ ((r/2)%8).  part =
 * scratch of the output projection (fp32 partial tiles, 512 x 256 KiB; its
 * contents after a call are unspecified).  n_pad is n_tokens rounded up to
 * 256.  Returns FLUX3_E_UNSUPPORTED for bad dims. */
typedef struct {
  size_t h, q, k, vt, cat, part, total;
  int64_t n_pad;
} flux3_workspace_layout;
flux3_status flux3_workspace_layout_get(const flux3_dims *dims, int64_t n_tokens,
                                        flux3_workspace_layout *out);

/* One transformer block, in place on the fp32 residual stream [P3 block
 * listing; P1; P4 "Inside the transformer"]:
 *   h   = (1 + scale_s) * LayerNorm(x) + shift_s     (no learned affine)
 *   q,k = RoPE(RMSNorm(h Wq^T)), RoPE(RMSNorm(h Wk^T)); v = h Wv^T
 *   out = Attention(q, k, v) Wo^T + (silu(h Wg^T) * (h Wu^T)) Wd^T
 *   x  += gate_s * out
 * where (shift_s, scale_s, gate_s) belong to the token's segment s; every
 * token attends to all n_tokens tokens.  A per-mode (stage-1) block is this
 * call on one stream's rows with a single segment.
 *   x    : device fp32 [n_tokens][width], updated in place.
 *   segs : host [n_segs], tiling [0, n_tokens) (see flux3_segment),
 *          1 <= n_segs <= FLUX3_MAX_SEGMENTS.
 *   mod  : device fp32 [n_segs][3][width] = shift, scale, gate per segment.
 *   rope : device fp32 [n_tokens][64][2] from flux3_rope_tables_build (or a
 *          row slice of one).
 *   workspace: device, >= flux3_workspace_bytes(dims, n_tokens) bytes.
 * n_tokens == 0 with n_segs == 0 is a no-op returning FLUX3_OK. */
flux3_status flux3_block_forward(const flux3_dims *dims,
                                 const flux3_block_weights *w, float *x,
                                 int64_t n_tokens, const flux3_segment *segs,
                                 int32_t n_segs, const float *mod,
                                 const float *rope, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * block of flux3_block_forward with the same arguments minus the
 * workspace.  Its intermediates (h, q, k, v^T, [o | act]) live in a device
 * array of FLUX3_NOALLOC_SCRATCH_BYTES bytes inside the library, one copy
 * per GPU, held from the first call on that GPU until the process ends;
 * the call itself allocates nothing.  n_tokens is limited to what fits --
 * 1024 tokens at width 3072, hidden 9216 -- and a larger call returns
 * FLUX3_E_WORKSPACE having enqueued nothing.  There is no split-partial
 * region, so the output GEMM and attention run every tile whole: slower
 * for small n_tokens than flux3_block_forward, and equal to it up to the
 * order of fp32 sums.  Calls that overlap on one GPU share the array and
 * race: serialise them (one stream, or events between streams).  The
 * first call on a device looks up the array's address there and returns
 * FLUX3_E_HIP if that fails.  Other errors as for flux3_block_forward. */
#define FLUX3_NOALLOC_SCRATCH_BYTES (48u * 1024u * 1024u)
flux3_status flux3_block_forward_noalloc(const flux3_dims *dims,
                                         const flux3_block_weights *w, float *x,
                                         int64_t n_tokens, const flux3_segment *segs,
                                         int32_t n_segs, const float *mod,
                                         const float *rope, void *stream);

/* The two-stage stack [P1; P4 "Inside the transformer"]:
 * stage 1 runs, for every segment s, the n_pm per-mode blocks of its mode
 * on that segment's rows alone (each stream attends only to itself);
 * stage 2 runs the n_joint joint blocks over all n_tokens with per-segment
 * modulation.  When the segments, each padded to 256 rows, fit the
 * workspace's rows (n_tokens rounded up to 256; true of [240 | 4096] and
 * [240 | 4096 | 4096]) and their modes' block-b weights share one layout,
 * stage 1 enqueues one launch sequence per block for all segments, each a
 * row group with its own weights and its own attention; otherwise one
 * sequence per segment.  Both give the same per-segment results (up to the
 * summation order of split output tiles).
 *   per_mode : host array [3 * n_pm]; block b of mode m is
 *              per_mode[m * n_pm + b] (entries of unused modes may be
 *              zeroed; they are only checked if a segment uses that mode).
 *   joint    : host array [n_joint].
 *   mod_stage1, mod_stage2 : device fp32; block b of a stage reads
 *              [n_segs][3][width] at offset b * mod_block_stride floats
 *              (stride 0 shares one set of vectors across the stage;
 *              a non-zero stride must be a multiple of 4).
 *   Other arguments as in flux3_block_forward. */
flux3_status flux3_stack_forward(const flux3_dims *dims,
                                 const flux3_block_weights *per_mode,
                                 int32_t n_pm,
                                 const flux3_block_weights *joint,
                                 int32_t n_joint, float *x, int64_t n_tokens,
                                 const flux3_segment *segs, int32_t n_segs,
                                 const float *mod_stage1,
                                 const float *mod_stage2,
                                 int64_t mod_block_stride, const float *rope,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);

/* ---------------------------------------------------------------------------
 * Modulation from timesteps.  Each block's adaLN (shift, scale, gate) comes
 * from the timestep embedding ("Speed, architecture, and how the tokens
 * move", 15jq.com post: image tokens take the current timestep, text and
 * reference tokens t = 0; "What step distillation removed",
 * rohitghumare.com guide: a 256 -> width -> width embedder with no biases,
 * and for the distilled flow map a second embedder of the target timestep
 * whose output is added; "The denoise loop", same guide: timesteps are
 * sigmas scaled by 1000):
 *   e(t)   = [cos(1000 t f_i), sin(1000 t f_i)],  f_i = 10000^(-i/128), i < 128
 *   E(t)   = W2 silu(W1 e(t));  E'(t) = W2' silu(W1' e(t))
 *   mod[s] = W_mod[mode_s] silu(E(t_mode_s) + E'(t_target))
 * split in the order shift, scale, gate.
 * ------------------------------------------------------------------------- */

/* Weights, bf16 in torch Linear layout [out][in]: the embedder w1
 * [width][256] and w2 [width][width]; the target embedder w1_tgt, w2_tgt
 * (same shapes; unused and may be NULL when t_target < 0); and one stage's
 * modulation linears w_mod[mode] [3*width][width] (mode 0 text, 1 image,
 * 2 reference; a mode no segment uses may be NULL). */
typedef struct {
  const void *w1, *w2, *w1_tgt, *w2_tgt;
  const void *w_mod[3];
} flux3_modulation_weights;

/* Workspace bytes flux3_modulation_forward needs: fp32 [4][256] + [8][width]
 * (an embedding, a hidden vector and E per timestep); 0 if dims are
 * unsupported. */
size_t flux3_modulation_workspace_bytes(const flux3_dims *dims);

/* One stage's modulation vectors for every segment.
 *   t_by_mode: host float[3], the timestep of each mode (text, image,
 *              reference); the model uses 0 for text and reference.  Values
 *              of the modes the segments use must be finite.
 *   t_target : the flow-map target timestep, or any negative value for none.
 *   segs     : host [n_segs], as for flux3_block_forward (tiling [0, N) in
 *              the order text, image, reference).
 *   mod      : device fp32 [n_segs][3][width] out, the layout
 *              flux3_block_forward and flux3_stack_forward take; segments of
 *              one mode get the same vectors.
 *   workspace: device, >= flux3_modulation_workspace_bytes(dims) bytes,
 *              256-byte aligned.
 * width must be <= 4096.  Matrix-vector work over the weights (about 190 MB
 * per call at width 3072), bound by HBM.  Errors as for flux3_block_forward;
 * on error nothing is enqueued. */
flux3_status flux3_modulation_forward(const flux3_dims *dims,
                                      const flux3_modulation_weights *w,
                                      const float *t_by_mode, float t_target,
                                      const flux3_segment *segs, int32_t n_segs,
                                      float *mod, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * One whole transformer call: the block stack with the linears around it
 * ("Speed, architecture, and how the tokens move", 15jq.com post: text
 * tokens as 20,480-value vectors, noisy image and reference tokens of 128
 * values, text and references dropped at the end; "The text encoder", "The
 * latent space and the VAE", "Inside the transformer", rohitghumare.com
 * guide: a linear to width 3072 for the text, an output linear from 3072
 * back to 128; no biases anywhere):
 *   x      = [text W_text^T | image W_img_in^T | refs W_ref_in^T]   (fp32)
 *   mod_1, mod_2 = each stage's modulation from t (image) and 0 (text,
 *            references), plus the target embedding when t_target >= 0
 *   x      = stack(x)                            (flux3_stack_forward)
 *   (shift, scale) = W_final silu(E(t) + E'(t_target))
 *   v      = ((1 + scale) LayerNorm(x_image) + shift) W_out^T
 * The inputs are rounded to bf16, the GEMM operand type, on the device; the
 * residual stream and the velocity are fp32.
 * ------------------------------------------------------------------------- */

/* Token vector sizes at the call's edges: text_dim = 20480 (8 stacked
 * 2,560-value text-encoder states), latent_dim = 128 (one 2x2 patch of the
 * 32-channel latent).  text_dim % 64 == 0 and text_dim <= 262144;
 * latent_dim % 64 == 0 and latent_dim <= 256. */
typedef struct {
  int32_t text_dim;
  int32_t latent_dim;
} flux3_io_dims;

/* The linears around the stack, bf16 in torch Linear layout [out][in]:
 *   w_text   [width][text_dim]     (may be NULL without text tokens)
 *   w_img_in [width][latent_dim]
 *   w_ref_in [width][latent_dim]   (may be NULL without reference tokens;
 *                                   pass w_img_in to share one input linear)
 *   w_final  [2 width][width]      output layer (shift, scale)
 *   w_out    [latent_dim][width] */
typedef struct {
  const void *w_text, *w_img_in, *w_ref_in, *w_final, *w_out;
} flux3_io_weights;

/* Workspace bytes flux3_transformer_forward needs for n_tokens tokens: the
 * block workspace (flux3_workspace_bytes) plus the fp32 residual stream,
 * the bf16 input staging, the modulation vectors and their workspace; 0 if
 * dims are unsupported. */
size_t flux3_transformer_workspace_bytes(const flux3_dims *dims, const flux3_io_dims *io_dims,
                                         int64_t n_tokens);

/* One transformer call; writes the velocity of the image tokens.
 *   mod_w   : host [2]: stage 1 and stage 2 modulation weights (see
 *             flux3_modulation_weights); the output layer uses stage 2's
 *             embedder (w1, w2 and, with a target, w1_tgt, w2_tgt).
 *   per_mode, n_pm, joint, n_joint: the blocks, as for flux3_stack_forward.
 *   text    : device bf16 [n_text][text_dim] (the rows of the mode-0
 *             segment; NULL if there is none).
 *   image   : device fp32 [n_image][latent_dim], the noisy latent tokens.
 *   refs    : device fp32 [n_ref][latent_dim], the reference tokens of all
 *             mode-2 segments in order (NULL if there are none).
 *   segs    : host; at most one text segment, exactly one image segment,
 *             then any reference segments, tiling [0, n_tokens).
 *   t       : the image timestep (sigma in [0, 1]); t_target < 0 for the
 *             base model, else the flow-map target timestep.
 *   rope    : device fp32 [n_tokens][64][2] for the call's layout.
 *   velocity: device fp32 [n_image][latent_dim] out.
 *   workspace: device, >= flux3_transformer_workspace_bytes, 256-byte
 *             aligned.
 * Errors as for flux3_stack_forward and flux3_modulation_forward; on error
 * nothing is enqueued. */
flux3_status flux3_transformer_forward(const flux3_dims *dims, const flux3_io_dims *io_dims,
                                       const flux3_io_weights *io,
                                       const flux3_modulation_weights *mod_w,
                                       const flux3_block_weights *per_mode, int32_t n_pm,
                                       const flux3_block_weights *joint, int32_t n_joint,
                                       const void *text, const float *image, const float *refs,
                                       const flux3_segment *segs, int32_t n_segs, float t,
                                       float t_target, const float *rope, float *velocity,
                                       void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * The denoise loop ("The denoise loop" and "What step distillation removed",
 * rohitghumare.com guide): steps noise levels evenly spaced from 1 down to
 * 1/steps, each shifted as sigma' = shift sigma / (1 + (shift - 1) sigma)
 * (shift 6.93 in the pipeline), then a final 0.  Each step calls the
 * transformer at sigma_i (the distilled flow map is also told sigma_{i+1})
 * and moves the latent by (sigma_{i+1} - sigma_i) v; latent - sigma_i v is
 * the step's preview of the clean latent.
 * ------------------------------------------------------------------------- */

/* The schedule into host sigmas[steps + 1] (computed in double, stored as
 * float).  Errors: FLUX3_E_SHAPE (steps < 1), FLUX3_E_INVALID (null or a
 * shift that is not positive and finite). */
flux3_status flux3_sigmas(int32_t steps, double shift, float *sigmas);

/* One step on n fp32 values (n % 4 == 0, device pointers 16-byte aligned):
 * x0_preview (optional, may be NULL) = latent - sigma v, then latent +=
 * (sigma_next - sigma) v.  Asynchronous on stream. */
flux3_status flux3_euler_step(const float *v, float *latent, float *x0_preview, int64_t n,
                              float sigma, float sigma_next, void *stream);

/* Workspace bytes flux3_sample needs: flux3_transformer_workspace_bytes
 * plus one velocity buffer; 0 if dims are unsupported. */
size_t flux3_sample_workspace_bytes(const flux3_dims *dims, const flux3_io_dims *io_dims,
                                    int64_t n_tokens);

/* The whole loop: steps transformer calls and Euler steps, all enqueued on
 * stream (no host synchronisation).
 *   latent   : device fp32 [n_image][latent_dim]: the starting noise in, the
 *              final latent out.
 *   distilled: non-zero to pass sigma_{i+1} as the target timestep (needs
 *              the target embedders in mod_w).
 *   previews : device fp32 [steps][n_image][latent_dim] out, or NULL.
 *   Other arguments as for flux3_transformer_forward (image is latent).
 * Errors as for flux3_transformer_forward and flux3_sigmas; on error
 * nothing is enqueued. */
flux3_status flux3_sample(const flux3_dims *dims, const flux3_io_dims *io_dims,
                          const flux3_io_weights *io, const flux3_modulation_weights *mod_w,
                          const flux3_block_weights *per_mode, int32_t n_pm,
                          const flux3_block_weights *joint, int32_t n_joint, const void *text,
                          float *latent, const float *refs, const flux3_segment *segs,
                          int32_t n_segs, int32_t steps, double shift, int32_t distilled,
                          const float *rope, float *previews, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Kernel timing, for benchmarks and profiling.  While enabled, every kernel
 * launch is bracketed by a pair of HIP events recorded on the launch stream,
 * so the durations are those of the kernels themselves on the stream they
 * run on.  flux3_profile_read waits for the recorded events and returns, for
 * one kernel kind, the number of launches, their summed duration in
 * milliseconds, and the summed token count M and M^2 of those launches (the
 * units the kernels' algorithmic work is counted in).  flux3_profile_reset
 * waits for and drops all records.  Records belong to the calling thread:
 * enable, the profiled calls, read and reset must come from one thread, and
 * other threads are unaffected.  Off by default.
 * This facility is the one exception to the library keeping nothing across
 * calls: while profiling is on, every launch creates two HIP events (host
 * runtime objects, no device buffers), held in the thread's records until
 * flux3_profile_reset destroys them. */
enum {
  FLUX3_K_ROPE_TABLES = 0,
  FLUX3_K_LN_MODULATE = 1,
  FLUX3_K_GEMM_PROJ = 2,
  FLUX3_K_ATTENTION = 3,
  FLUX3_K_GEMM_OUT = 4,
  FLUX3_K_MODULATION = 5,   /* one record per flux3_modulation_forward call */
  FLUX3_K_IO_LINEARS = 6,   /* each input / output linear of a transformer call */
  FLUX3_K_EULER = 7,        /* each flux3_euler_step (and sampler step update) */
  FLUX3_K_QUANT = 8,        /* per-token e4m3 quantisation of [o | act] (FP8R blocks) */
  FLUX3_K_COUNT = 9
};
typedef struct {
  int64_t launches;
  double total_ms;
  double tokens;     /* sum of M over launches   */
  double tokens_sq;  /* sum of M*M over launches; an attention launch over
                        several equal-length streams adds each stream's M*M */
} flux3_kernel_stats;
void flux3_profile_enable(int32_t on);
void flux3_profile_reset(void);
/* FLUX3_E_INVALID for a bad kind or NULL out; FLUX3_E_HIP if an event
 * cannot be read. */
flux3_status flux3_profile_read(int32_t kernel, flux3_kernel_stats *out);
/* As flux3_profile_read, over the launches of that kind whose token count
 * M equals n_tokens (a block's joint launches apart from its per-stream
 * ones, say).  FLUX3_E_SHAPE for a negative n_tokens. */
flux3_status flux3_profile_read_tokens(int32_t kernel, int64_t n_tokens,
                                       flux3_kernel_stats *out);

/* What the kernels run on: compute units and shader clock of a HIP device,
 * its architecture name, and the dense bf16 MFMA peak those imply for the
 * gfx950 matrix cores (4096 FLOP per clock per CU): CUs x clock x 4096.
 * FLUX3_E_INVALID for a NULL out, FLUX3_E_HIP if the device cannot be
 * queried.  Host-only; enqueues nothing. */
typedef struct {
  int32_t compute_units;
  int32_t clock_khz;          /* maximum shader clock */
  double bf16_dense_tflops;   /* compute_units * clock * 4096 / 1e12 */
  char arch[64];              /* e.g. "gfx950:sramecc+:xnack-" */
} flux3_device_info;
flux3_status flux3_device_query(int32_t device, flux3_device_info *out);

/* Debug switch: when non-zero every launch is followed by a stream
 * synchronisation and an error check, so a faulting kernel is named in
 * flux3_last_error_detail().  Off by default. */
void flux3_set_debug_sync(int32_t on);

const char *flux3_status_string(flux3_status s);
const char *flux3_last_error_detail(void);

#ifdef __cplusplus
}
#endif
#endif /* FLUX3_H */
