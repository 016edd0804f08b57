// Measurement helper: a plain streaming read of device memory, the
// achievable-bandwidth reference that the decode kernels' HBM rates are
// compared with (the decode step is bound by weight and KV-cache reads:
// kongchang.com/en article, section "Why do Prefill and Decode need
// different quantization strategies?").
#include <hip/hip_runtime.h>

#include "internal.h"

namespace futx {

// Each workgroup reads one contiguous chunk with 128-bit loads, U loads per
// lane in flight; the XOR of everything read goes to sink[blockIdx] only when
// it equals a value no input here produces, which keeps the loads alive
// without a store per workgroup.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t x = 0;
  for (size_t i = b0 + threadIdx.x; i < b1; i += 256 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + (size_t)u * 256;
      v[u] = j < b1 ? p[j] : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (x == 0x9E3779B9u && threadIdx.x == 0) sink[blockIdx.x] = x;
}

}  // namespace futx

using namespace futx;

extern "C" {

futx_status futx_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream) {
  clear_error();
  if (!buf || !sink || bytes == 0 || (bytes & 15) || ((uintptr_t)buf & 15))
    return fail(FUTX_E_ARG, "stream_read: buffer must be non-null, 16-byte aligned, a positive multiple of 16 bytes");
  if (workgroups < 1 || workgroups > 65536) return fail(FUTX_E_ARG, "stream_read: workgroups must be 1..65536");
  stream_read_kernel<8><<<workgroups, 256, 0, (hipStream_t)stream>>>((const uint4*)buf, bytes / 16, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FUTX_E_HIP, "stream_read: %s", hipGetErrorString(e));
  return FUTX_OK;
}

}  // extern "C"
