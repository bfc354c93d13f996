// Host-side pieces of the C ABI shared between its source files.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/flux3.h"
#include "kernels.hpp"

namespace flux3 {

// Every check flux3_block_forward makes except the workspace; fills the
// segment table.  FLUX3_OK for n_tokens == 0 with n_segs == 0 (a no-op).
flux3_status validate_block(const flux3_dims* dims, const flux3_block_weights* w, const float* x,
                            int64_t n_tokens, const flux3_segment* segs, int32_t n_segs,
                            const float* mod, const float* rope, SegTableHost* st);

// Bytes of a block's intermediate buffers (h, q, k, vt, cat) for n_tokens:
// the workspace without its split-partial region.  dims must be valid.
size_t block_buffer_bytes(const flux3_dims* dims, int64_t n_tokens);

// Enqueues one validated block with `buffers` (>= block_buffer_bytes) as
// its intermediates and no split-partial region: the output GEMM and
// attention run every tile whole.
flux3_status run_block_whole_tiles(const flux3_dims* dims, const flux3_block_weights* w, float* x,
                                   int64_t n_tokens, const SegTableHost& st, const float* mod,
                                   const float* rope, void* buffers, void* stream);

// Sets the per-thread detail message flux3_last_error_detail() returns.
flux3_status set_error(flux3_status s, const char* fmt, ...);

}  // namespace flux3
