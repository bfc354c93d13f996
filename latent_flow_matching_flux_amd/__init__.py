"""MI355X (gfx950) forward path of the FLUX.3 Image Klein transformer block.

The computation lives in libflux3.so (HIP kernels behind the C ABI in
include/flux3.h); this package holds the build script and a thin ctypes
binding with the same entry-point names.
"""
from ._lib import (Flux3Error, Dims, Segment, BlockWeights, RopeLayout, WorkspaceLayout,
                   load, layout_tokens, rope_tables_build, workspace_bytes, workspace_layout,
                   block_forward, block_forward_noalloc, NOALLOC_SCRATCH_BYTES, stack_forward,
                   set_debug_sync, status_string, EXPORTS,
                   LIB_PATH, KERNELS, profile_enable, profile_reset, profile_read,
                   device_query, modulation_workspace_bytes, modulation_forward,
                   ModulationWeights, weights_packed_bytes, weights_pack, WEIGHTS_LINEAR,
                   WEIGHTS_PACKED, WEIGHTS_FP8R, weights_fp8r_bytes, weights_quantize_fp8r,
                   IoDims, IoWeights, transformer_workspace_bytes,
                   transformer_forward, sigmas, euler_step, sample_workspace_bytes, sample)

__all__ = ["Flux3Error", "Dims", "Segment", "BlockWeights", "RopeLayout", "WorkspaceLayout",
           "load", "layout_tokens", "rope_tables_build", "workspace_bytes", "workspace_layout",
           "block_forward", "block_forward_noalloc", "NOALLOC_SCRATCH_BYTES", "stack_forward",
           "set_debug_sync", "status_string", "EXPORTS",
           "LIB_PATH", "KERNELS", "profile_enable", "profile_reset", "profile_read",
           "device_query", "modulation_workspace_bytes", "modulation_forward",
           "ModulationWeights", "weights_packed_bytes", "weights_pack", "WEIGHTS_LINEAR",
           "WEIGHTS_PACKED", "WEIGHTS_FP8R", "weights_fp8r_bytes", "weights_quantize_fp8r",
           "IoDims", "IoWeights", "transformer_workspace_bytes",
           "transformer_forward", "sigmas", "euler_step", "sample_workspace_bytes", "sample"]
