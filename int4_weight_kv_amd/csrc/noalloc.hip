// futx_decode_block_noalloc: the decode block with a library-owned static
// device workspace, for callers that cannot allocate (code under graph
// capture, tight serving loops, harnesses that forbid hipMalloc).  It runs
// the same kernels, in the same order and launch configuration, as
// futx_decode_block.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace futx {

// The workspace: a file-scope device array, one copy on each GPU the library
// is loaded on, held until the process ends.  Host code never uses its name
// as an address: the device address comes from hipGetSymbolAddress, once per
// device, with that device current.  Nothing in it needs to start at zero
// (every buffer a kernel reads was written earlier in the same call), and
// every call on a GPU shares that GPU's copy, so calls that overlap on one
// GPU (other streams, other threads) race.
constexpr size_t kScratchBytes = (size_t)72 << 20;  // covers 70B-shape blocks at batch 32
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device (looked up on the first
// call for that device).
static futx_status scratch_address(void** out) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {nullptr};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FUTX_E_HIP, "decode_block_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FUTX_E_UNSUPPORTED, "decode_block_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FUTX_E_HIP, "decode_block_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return FUTX_OK;
}

}  // namespace futx

using namespace futx;

extern "C" {

futx_status futx_decode_block_noalloc(const futx_dims* dims, const futx_block_weights* w, int32_t batch,
                                      float* x, const int32_t* cached_lens, const int32_t* block_table,
                                      int32_t max_pages_per_seq, int32_t max_context,
                                      const futx_kv_cache* cache, void* stream) {
  clear_error();
  futx_status st = check_dims(dims);
  if (st) return st;
  if (batch < 1 || batch > kMaxBatch) return fail(FUTX_E_ARG, "decode_block_noalloc: batch must be 1..32");
  if (max_context < 1) return fail(FUTX_E_ARG, "decode_block_noalloc: max_context must be positive");
  const size_t need = decode_workspace_bytes(*dims, batch, max_context);
  if (need > kScratchBytes)
    return fail(FUTX_E_WORKSPACE,
                "decode_block_noalloc: batch %d and max_context %d need %zu bytes of scratch; the static buffer "
                "holds %zu (use futx_decode_block with a workspace)",
                (int)batch, (int)max_context, need, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return decode_block_impl(dims, w, batch, x, cached_lens, block_table, max_pages_per_seq, max_context, cache, ws,
                           kScratchBytes, stream, -1);
}

}  // extern "C"
