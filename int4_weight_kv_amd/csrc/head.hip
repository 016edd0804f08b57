// Full decode step around the blocks: token embedding, and the LM head with
// the final RMSNorm (gain folded into the bf16 head weights, as the pages
// fold the fixed norm gains into the weights that follow a norm: FP8 Prefill
// + INT4 Decode article, section "FP8 Prefill: fusing GEMM and epilogue all
// the way") and the top-1 token.
//
// The LM head is a bf16 matrix-vector product over vocab x hidden weights
// (1.05 GB for Llama-3.1-8B), bound by HBM bandwidth.  Four kernels:
//   prep    u = bf16(x), 1/r per row                       (prep_act_kernel)
//   partial the K range in slices of 1024; a 4-wave workgroup stages its bf16 u
//           slice in LDS, each wave streams one 16-row vocab tile through the
//           bf16 matrix cores (weights as the B operand, straight from HBM)
//           and writes fp32 partial sums; it also clears the top-1 keys
//   reduce  logits = (sum of the partials, fixed order) / r, and a 64-bit
//           atomic max of (order-preserving value, inverted index) per row:
//           the largest logit, lowest index on ties, independent of order
//   top1    decodes the keys
#include "device.h"
#include "head.h"
#include "kernels.h"

namespace futx {

constexpr int kHeadChunk = 8;  // MFMA steps (32 inputs each) per load chunk (256 inputs)

// K splits of the LM head: slices of 1024 inputs, or one split
static int head_splits(int H) { return H % 1024 == 0 ? H / 1024 : 1; }

__global__ __launch_bounds__(256) void embed_kernel(const uint16_t* __restrict__ table, const int32_t* tokens,
                                                    int vocab, int H, float* __restrict__ x) {
  const int b = blockIdx.x;
  int t = tokens[b];
  t = t < 0 ? 0 : (t >= vocab ? vocab - 1 : t);  // device metadata is trusted; stay in bounds anyway
  const uint16_t* row = table + (size_t)t * H;
  for (int c = threadIdx.x; c < H; c += 256) x[(size_t)b * H + c] = bf16_bits_to_f32(row[c]);
}

// Batch placement as in the INT4 GEMM: A row `col` holds batch
// 4 (col % 4) + col / 4 (rows past the batch repeat row 0), so D register r
// of lane group grp holds batch 4r + grp.
template <int NR>
__global__ __launch_bounds__(256, 2) void lm_head_partial_kernel(const uint16_t* __restrict__ w,
                                                                 const uint16_t* __restrict__ u, int B,
                                                                 int H, int V, int ks, float* __restrict__ part,
                                                                 unsigned long long* __restrict__ keys) {
  extern __shared__ __align__(16) uint8_t s_dyn[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wq = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int split = blockIdx.y;
  const int kr = H / ks;  // inputs of this split (a multiple of 256)
  const int k0 = split * kr;
  const int row = kr + 8;  // bf16 per LDS row (16 B pad)
  uint16_t* const s_u = (uint16_t*)s_dyn;
  if (blockIdx.x == 0 && split == 0 && tid < B) keys[tid] = 0ull;
  // stage the u slice: B rows x kr bf16
  for (int i = tid; i < B * (kr / 8); i += 256) {
    const int b = i / (kr / 8), c8 = i - b * (kr / 8);
    *(uint4*)(s_u + (size_t)b * row + c8 * 8) = *(const uint4*)(u + (size_t)b * H + k0 + c8 * 8);
  }
  __syncthreads();
  const int tile = blockIdx.x * 4 + wq;  // 16 vocab rows
  if (tile * 16 >= V) return;            // whole wave (uniform); no barrier follows
  int bb = 4 * (col & 3) + (col >> 2);
  if (bb >= B) bb = 0;
  const uint8_t* const a_base = (const uint8_t*)(s_u + (size_t)bb * row + grp * 8);
  int vr = tile * 16 + col;
  if (vr >= V) vr = V - 1;  // rows past the vocabulary re-read the last row, unused
  const uint4* const wrow = (const uint4*)(w + (size_t)vr * H + k0 + grp * 8);
  const int nsteps = kr / 32;  // MFMA steps
  const int nchunks = nsteps / kHeadChunk;
  uint4 wa[kHeadChunk], wb[kHeadChunk];
  auto load = [&](uint4 (&r)[kHeadChunk], int c) {
#pragma unroll
    for (int s = 0; s < kHeadChunk; ++s) r[s] = wrow[(c * kHeadChunk + s) * 4];  // 32 bf16 = 4 uint4 per step
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const uint4 (&r)[kHeadChunk], int c) {
#pragma unroll
    for (int s = 0; s < kHeadChunk; ++s) {
      const bf16x8 av = *(const bf16x8*)(a_base + (size_t)(c * kHeadChunk + s) * 64);
      acc = mfma16(av, as_bf16x8(r[s]), acc);
    }
  };
  // two chunks in flight; every load in the loop is unconditional
  load(wa, 0);
  load(wb, nchunks > 1 ? 1 : 0);
  int c = 0;
  for (; c + 3 < nchunks; c += 2) {
    compute(wa, c);
    load(wa, c + 2);
    compute(wb, c + 1);
    load(wb, c + 3);
  }
  compute(wa, c);
  if (c + 2 < nchunks) load(wa, c + 2);
  if (c + 1 < nchunks) compute(wb, c + 1);
  if (c + 2 < nchunks) compute(wa, c + 2);
  if (tile * 16 + col < V) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int b = 4 * r + grp;
      if (b < B) part[((size_t)split * B + b) * V + tile * 16 + col] = acc[r];
    }
  }
}

__device__ __forceinline__ unsigned long long top1_key(float v, int idx) {
  uint32_t bits = __float_as_uint(v);
  bits = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);  // order-preserving
  return ((unsigned long long)bits << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}

__global__ __launch_bounds__(256) void lm_head_reduce_kernel(const float* __restrict__ part, const float* invr,
                                                             int B, int V, int ks, float* __restrict__ logits,
                                                             unsigned long long* keys) {
  const int b = blockIdx.y;
  const float s = invr[b];
  unsigned long long best = 0ull;
  for (int v = blockIdx.x * 256 + threadIdx.x; v < V; v += gridDim.x * 256) {
    float t = 0.f;
    for (int k = 0; k < ks; ++k) t += part[((size_t)k * B + b) * V + v];
    const float l = t * s;
    logits[(size_t)b * V + v] = l;
    const unsigned long long key = top1_key(l, v);
    best = key > best ? key : best;
  }
  // wave max, then one atomic per wave
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long other = __shfl_xor(best, o, 64);
    best = other > best ? other : best;
  }
  if ((threadIdx.x & 63) == 0) atomicMax(&keys[b], best);
}

__global__ void top1_kernel(const unsigned long long* keys, int B, int32_t* top1) {
  const int b = threadIdx.x;
  if (b < B) top1[b] = (int32_t)(0xFFFFFFFFu - (uint32_t)(keys[b] & 0xFFFFFFFFull));
}

HeadWs head_ws(int hidden, int vocab, int max_batch, char* base) {
  HeadWs w{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + at : nullptr;
    at += (bytes + 255) & ~(size_t)255;
    return p;
  };
  w.u = (uint16_t*)take((size_t)max_batch * hidden * 2);
  w.invr = (float*)take((size_t)max_batch * 4);
  w.part = (float*)take((size_t)head_splits(hidden) * (max_batch < 16 ? max_batch : 16) * vocab * 4);
  w.keys = (unsigned long long*)take((size_t)max_batch * 8);
  w.bytes = at;
  return w;
}

bool head_shape_ok(int hidden) { return hidden > 0 && hidden % (32 * kHeadChunk) == 0; }

hipError_t launch_embed(const uint16_t* table, const int32_t* tokens, int vocab, int H, int B, float* x,
                        hipStream_t st) {
  embed_kernel<<<B, 256, 0, st>>>(table, tokens, vocab, H, x);
  return hipGetLastError();
}

// rows [b0, b0 + nb) of the batch, nb <= 16
static hipError_t lm_head_rows(const uint16_t* w, const float* x, int nb, int H, int V, float eps,
                               const HeadWs& ws, float* logits, int32_t* top1, hipStream_t st) {
  hipError_t e = launch_prep_act(x, nb, H, eps, ws.u, ws.invr, st);
  if (e != hipSuccess) return e;
  const int ks = head_splits(H);
  const int tiles = (V + 15) / 16;
  const dim3 grid((tiles + 3) / 4, ks);
  const size_t lds = (size_t)nb * (H / ks + 8) * 2;
  auto k1 = lm_head_partial_kernel<1>, k2 = lm_head_partial_kernel<2>, k4 = lm_head_partial_kernel<4>;
  auto k = nb <= 4 ? k1 : (nb <= 8 ? k2 : k4);
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  k<<<grid, 256, lds, st>>>(w, ws.u, nb, H, V, ks, ws.part, ws.keys);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  lm_head_reduce_kernel<<<dim3(64, nb), 256, 0, st>>>(ws.part, ws.invr, nb, V, ks, logits, ws.keys);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  top1_kernel<<<1, 64, 0, st>>>(ws.keys, nb, top1);
  return hipGetLastError();
}

hipError_t launch_lm_head(const uint16_t* w, const float* x, int B, int H, int V, float eps, const HeadWs& ws,
                          float* logits, int32_t* top1, hipStream_t st) {
  // batches above 16 run as halves of at most 16 rows (one matrix-core fragment)
  for (int b0 = 0; b0 < B; b0 += 16) {
    const int nb = B - b0 < 16 ? B - b0 : 16;
    hipError_t e = lm_head_rows(w, x + (size_t)b0 * H, nb, H, V, eps, ws, logits + (size_t)b0 * V, top1 + b0, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace futx
