// flux3_block_forward_noalloc: flux3_block_forward with its intermediates in
// a fixed device array of the library instead of a caller workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` below exists once per GPU the library runs on and is
// held until the process ends.  Host code never passes its name to a kernel
// (on the host it only stands for the device symbol): the first call on a
// device looks up that device's address of it with hipGetSymbolAddress, with
// the device current, and every call uses that address.  Nothing in the
// block needs the buffers zeroed (each call writes every element it reads),
// so the previous call's contents are harmless.  Calls that overlap on one
// GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "abi_internal.hpp"

namespace {

constexpr int kMaxDevices = 64;

// The block's intermediate buffers (h, q, k, v^T, [o | act]) for up to
// FLUX3_NOALLOC_SCRATCH_BYTES bytes: 1024 tokens at width 3072 / hidden 9216.
static __device__ __align__(256) unsigned char scratch[FLUX3_NOALLOC_SCRATCH_BYTES];

void* g_scratch[kMaxDevices];
hipError_t g_setup[kMaxDevices];
std::once_flag g_once[kMaxDevices];

}  // namespace

extern "C" flux3_status flux3_block_forward_noalloc(const flux3_dims* dims,
                                                    const flux3_block_weights* w, float* x,
                                                    int64_t n_tokens, const flux3_segment* segs,
                                                    int32_t n_segs, const float* mod,
                                                    const float* rope, void* stream) {
  flux3::SegTableHost st;
  flux3_status r = flux3::validate_block(dims, w, x, n_tokens, segs, n_segs, mod, rope, &st);
  if (r != FLUX3_OK || n_tokens == 0) return r;
  const size_t need = flux3::block_buffer_bytes(dims, n_tokens);
  if (need > sizeof(scratch))
    return flux3::set_error(FLUX3_E_WORKSPACE,
                            "n_tokens %lld needs %zu bytes of intermediates; the allocation-free "
                            "entry point holds %zu (use flux3_block_forward with a workspace)",
                            (long long)n_tokens, need, sizeof(scratch));
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return flux3::set_error(FLUX3_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return flux3::set_error(FLUX3_E_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::call_once(g_once[dev], [dev] {
    g_setup[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
  });
  if (g_setup[dev] != hipSuccess || !g_scratch[dev])
    return flux3::set_error(FLUX3_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                            hipGetErrorString(g_setup[dev]));
  return flux3::run_block_whole_tiles(dims, w, x, n_tokens, st, mod, rope, g_scratch[dev], stream);
}
