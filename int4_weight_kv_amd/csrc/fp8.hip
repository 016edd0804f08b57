// FP8 (e4m3) weight-and-activation variant of the decode projection on the
// gfx950 fp8 matrix cores: the comparison point the pages set the INT4
// decode path against (the INT4 decode block is 31-51% faster than the
// authors' FP8 path: FuTransformer abstract, airebao.com item page).
//
// Format (a reading; the pages give none): OCP e4m3 "fn" bytes (bias 7,
// largest finite 448, 0x7F NaN), one fp32 scale per group of 128 inputs for
// weight rows and for activation rows, s = fp32(max|x| / 448), codes
// e4m3(fp32(x / s)) rounded to nearest even and saturated at 448.
//
// Weight layout: packed[nt][kb][lane 64][32 bytes]: lane L holds row
// nt * 16 + L % 16, and byte 8 s + e holds input kb * 128 + 32 s + 8 (L / 16)
// + e, the B operand of v_mfma_f32_16x16x32_fp8_fp8 for MFMA step s (two
// 128-bit loads per lane per 128 inputs); scales fp32 [nt][kb][16].  Rows
// are in logical order (gate rows then up rows for GATEUP).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "device.h"
#include "gemm.h"
#include "internal.h"
#include "kernels.h"

namespace futx {

constexpr int kFp8Group = 128;
constexpr float kE4m3Max = 448.0f;

// e4m3fn byte of an fp32 value: round to nearest even, saturate at +-448.
// For |v| = f 2^x (f in [0.5, 1)) the code's exponent is E = x - 1 clamped
// to [-6, 8]; q = rint(|v| 2^(3 - E)) counts steps of 2^(E - 3) (exact
// power-of-two scaling); q = 16 carries into the next exponent; q < 8 (only
// at E = -6) is a subnormal.  The same fp32 operations on host and device.
__host__ __device__ inline uint8_t e4m3_encode(float v) {
  const float a = fabsf(v);
  int x = 0;
  (void)frexpf(a, &x);
  int E = x - 1;
  E = E < -6 ? -6 : (E > 8 ? 8 : E);
  float q = rintf(ldexpf(a, 3 - E));
  if (q >= 16.0f) {
    ++E;
    q *= 0.5f;
  }
  uint32_t code;
  if (E > 8 || (E == 8 && q > 14.0f)) code = 0x7E;
  else if (q >= 8.0f) code = (uint32_t)(((E + 7) << 3) | ((int)q - 8));
  else code = (uint32_t)q;
  if (__builtin_bit_cast(uint32_t, v) >> 31) code |= 0x80u;  // sign bit (negative zero too)
  return (uint8_t)code;
}

// ---------------------------------------------------------------- packer

static void fp8_pack_rows(const float* w, const float* gain, int K, int r0, int r1, uint8_t* packed,
                          float* scales) {
  const int KB = K / kFp8Group;
  std::vector<float> row(K);
  for (int n = r0; n < r1; ++n) {
    const float* src = w + (size_t)n * K;
    for (int c = 0; c < K; ++c) row[c] = gain ? src[c] * gain[c] : src[c];
    const int nt = n / 16, i = n % 16;
    for (int kb = 0; kb < KB; ++kb) {
      const float* xg = row.data() + (size_t)kb * kFp8Group;
      float a = 0.f;
      for (int c = 0; c < kFp8Group; ++c) a = std::fmax(a, std::fabs(xg[c]));
      const float s = a / kE4m3Max;
      scales[((size_t)nt * KB + kb) * 16 + i] = s;
      for (int c = 0; c < kFp8Group; ++c) {
        const float r = s == 0.f ? 0.f : xg[c] / s;
        const int st = c / 32, g = (c % 32) / 8, e = c % 8;
        const int lane = g * 16 + i;
        packed[(((size_t)nt * KB + kb) * 64 + lane) * 32 + st * 8 + e] = e4m3_encode(r);
      }
    }
  }
}

static futx_status fp8_shape(const futx_dims* dims, futx_proj proj, ProjShape* ps) {
  futx_status st = check_dims(dims);
  if (st || (st = check_proj(proj))) return st;
  *ps = proj_shape(*dims, proj);
  if (ps->k % kFp8Group || ps->n % 16) return fail(FUTX_E_UNSUPPORTED, "fp8: shape not a multiple of 128 x 16");
  return FUTX_OK;
}

// ---------------------------------------------------------------- kernels

// Activation rows bf16 [B][K] -> e4m3 codes [B][K] and fp32 scales
// [B][K / 128]: one wave per (group, row), two inputs per lane.
__global__ __launch_bounds__(64) void fp8_quant_act_kernel(const uint16_t* __restrict__ act, int K,
                                                           uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int g = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const size_t base = (size_t)b * K + (size_t)g * kFp8Group;
  const float x0 = bf16_bits_to_f32(act[base + lane]), x1 = bf16_bits_to_f32(act[base + 64 + lane]);
  const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float s = amax / kE4m3Max;
  codes[base + lane] = e4m3_encode(s == 0.f ? 0.f : x0 / s);
  codes[base + 64 + lane] = e4m3_encode(s == 0.f ? 0.f : x1 / s);
  if (lane == 0) scales[(size_t)b * (K / kFp8Group) + g] = s;
}

struct Fp8Args {
  const uint4* w;      // packed weights
  const float* sw;     // weight scales [nt][kb][16]
  const uint8_t* act;  // activation codes [B][K]
  const float* sa;     // activation scales [B][K / 128]
  float* out;          // [splits][B][N]
  int N, K, B;
  int kb_per_split, items, wgs_per_split;
};

// A workgroup of 4 waves owns a run of 16-row items over one K range; each
// wave owns a quarter of that range for every item.  A wave stages its
// quarter of the activation codes and scales (all rows) in LDS (it reads only
// what it wrote: no barrier), then streams its weights in chunks of 4 K
// blocks (8 KB per wave) with the next chunk in flight.  Per K block (one
// scale group): d = sum over 4 fp8 MFMA steps, acc += s_w s_a d.  The wave
// sums of an item are added in LDS (fixed order) at the end of the item.
// Batch b sits in A row b % 16 of fragment b / 16; rows past the batch read
// row 0 and are never written out.
template <int NF>
__global__ __launch_bounds__(256) void fp8_gemm_kernel(Fp8Args a) {
  constexpr int CHK = 4;
  extern __shared__ __align__(16) uint8_t s_dyn[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wq = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int B = a.B, KB = a.K / kFp8Group;
  const int split = blockIdx.x / a.wgs_per_split, wj = blockIdx.x - split * a.wgs_per_split;
  const int kb0 = split * a.kb_per_split, kb1 = min(kb0 + a.kb_per_split, KB);
  const int krange = kb1 - kb0;
  const int it0 = (int)((long)wj * a.items / a.wgs_per_split);
  const int it1 = (int)((long)(wj + 1) * a.items / a.wgs_per_split);
  const int kbq = (krange + 3) / 4;
  const int q0 = min(kb0 + wq * kbq, kb1), q1 = min(q0 + kbq, kb1);
  const int row = krange * kFp8Group + 16;  // LDS bytes per activation row (16 B pad)
  uint8_t* const s_act = s_dyn;
  float* const s_sa = (float*)(s_dyn + (((size_t)B * row + 15) & ~(size_t)15));
  float* const s_part = s_sa + ((B * krange + 3) & ~3);
  if (it0 >= it1) return;  // whole workgroup, before any barrier

  // stage this wave's quarter of the activation codes and scales
  for (int idx = lane; idx < B * (q1 - q0) * 8; idx += 64) {
    const int b = idx / ((q1 - q0) * 8), c16 = idx - b * (q1 - q0) * 8;
    const size_t k = (size_t)q0 * kFp8Group + (size_t)c16 * 16;
    *(uint4*)(s_act + (size_t)b * row + (k - (size_t)kb0 * kFp8Group)) = *(const uint4*)(a.act + (size_t)b * a.K + k);
  }
  for (int idx = lane; idx < B * (q1 - q0); idx += 64) {
    const int b = idx / (q1 - q0), j = idx - b * (q1 - q0);
    s_sa[b * krange + (q0 - kb0) + j] = a.sa[(size_t)b * KB + q0 + j];
  }

  const int nq = q1 - q0;                   // K blocks of this wave per item
  const int cpi = (kbq + CHK - 1) / CHK;    // chunks per item (same for every wave)
  const int nchunks = (it1 - it0) * cpi;
  uint4 wA[CHK][2], wB[CHK][2];
  float sA[CHK], sB[CHK];
  auto load = [&](uint4 (&w)[CHK][2], float (&sc)[CHK], int c) {
    const int item = it0 + c / cpi, cb = q0 + (c % cpi) * CHK;
#pragma unroll
    for (int i = 0; i < CHK; ++i) {
      const int kb = cb + i < q1 ? cb + i : (nq > 0 ? q0 : kb0);  // past the quarter: a valid block, weighted 0
      const uint4* p = a.w + (((size_t)item * KB + kb) * 64 + lane) * 2;
      w[i][0] = p[0];
      w[i][1] = p[1];
      sc[i] = a.sw[((size_t)item * KB + kb) * 16 + col];
    }
  };
  int b_row[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) b_row[f] = 16 * f + col < B ? 16 * f + col : 0;
  f32x4 acc[NF];
  auto zero = [&]() {
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  zero();
  auto compute = [&](const uint4 (&w)[CHK][2], const float (&sc)[CHK], int c) {
    if (nq == 0) return;
    const int cb = q0 + (c % cpi) * CHK;
#pragma unroll
    for (int i = 0; i < CHK; ++i) {
      const bool live = cb + i < q1;
      const int kb = live ? cb + i : q0;
      f32x4 d[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) d[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 wv = w[i][s >> 1];
        const long bw = (s & 1) ? (long)(((uint64_t)wv.w << 32) | wv.z) : (long)(((uint64_t)wv.y << 32) | wv.x);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const long av = *(const long*)(s_act + (size_t)b_row[f] * row + (size_t)(kb - kb0) * kFp8Group + s * 32 + grp * 8);
          d[f] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(av, bw, d[f], 0, 0, 0);
        }
      }
      const float swv = live ? sc[i] : 0.f;
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int b = 16 * f + 4 * grp + r;
          const float sav = s_sa[(b < B ? b : 0) * krange + (kb - kb0)];
          acc[f][r] = fmaf(swv * sav, d[f][r], acc[f][r]);
        }
    }
  };
  auto finish = [&](int c) {
    if ((c + 1) % cpi) return;
    const int item = it0 + c / cpi;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_part[((wq * NF + f) * 4 + r) * 64 + lane] = acc[f][r];
    zero();
    __syncthreads();
    if (wq == (item - it0) % 4) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int b = 16 * f + 4 * grp + r;
          float o = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) o += s_part[((w * NF + f) * 4 + r) * 64 + lane];
          if (b < B) a.out[((size_t)split * B + b) * a.N + (size_t)item * 16 + col] = o;
        }
    }
    __syncthreads();
  };
  load(wA, sA, 0);
  if (nchunks > 1) load(wB, sB, 1);
  int c = 0;
  for (; c + 2 < nchunks; c += 2) {
    compute(wA, sA, c);
    load(wA, sA, c + 2);
    finish(c);
    compute(wB, sB, c + 1);
    if (c + 3 < nchunks) load(wB, sB, c + 3);
    finish(c + 1);
  }
  compute(wA, sA, c);
  finish(c);
  if (c + 1 < nchunks) {
    compute(wB, sB, c + 1);
    finish(c + 1);
  }
}

struct Fp8Plan {
  int splits, kb_per_split, wgs_per_split, items;
  size_t lds;
};

static size_t fp8_lds(int B, int krange) {
  const size_t act = ((size_t)B * (krange * kFp8Group + 16) + 15) & ~(size_t)15;
  const size_t sa = (size_t)((B * krange + 3) & ~3) * 4;
  const int nf = B <= 16 ? 1 : 2;
  return act + sa + (size_t)4 * nf * 4 * 64 * 4;
}

static Fp8Plan fp8_plan(int N, int K, int B) {
  Fp8Plan p{};
  const int KB = K / kFp8Group;
  p.splits = 1;
  // the staged activation range stays within 64 KB (two workgroups per CU)
  while (p.splits < KB && (long)B * ((KB + p.splits - 1) / p.splits) * kFp8Group > 64 * 1024) ++p.splits;
  p.kb_per_split = (KB + p.splits - 1) / p.splits;
  p.splits = (KB + p.kb_per_split - 1) / p.kb_per_split;
  p.items = N / 16;
  const int target = (2 * device_cu_count() + p.splits - 1) / p.splits;
  const int per = (p.items + target - 1) / target;
  p.wgs_per_split = (p.items + per - 1) / per;
  p.lds = fp8_lds(B, p.kb_per_split);
  return p;
}

struct Fp8Ws {
  uint8_t* codes;
  float* scales;
  float* part;
  size_t bytes;
};

static Fp8Ws fp8_ws(int N, int K, int B, char* base) {
  Fp8Ws w{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + at : nullptr;
    at += round_up(bytes, 256);
    return p;
  };
  const Fp8Plan p = fp8_plan(N, K, B);
  w.codes = (uint8_t*)take((size_t)B * K);
  w.scales = (float*)take((size_t)B * (K / kFp8Group) * 4);
  w.part = (float*)take(p.splits > 1 ? (size_t)p.splits * B * N * 4 : 4);
  w.bytes = at;
  return w;
}

}  // namespace futx

using namespace futx;

extern "C" {

futx_status futx_fp8_packed_sizes(const futx_dims* dims, futx_proj proj, size_t* packed_bytes, size_t* scale_bytes) {
  clear_error();
  ProjShape ps;
  futx_status st = fp8_shape(dims, proj, &ps);
  if (st) return st;
  if (!packed_bytes || !scale_bytes) return fail(FUTX_E_ARG, "fp8_packed_sizes: null output pointer");
  *packed_bytes = (size_t)ps.n * ps.k;
  *scale_bytes = (size_t)ps.n * (ps.k / kFp8Group) * 4;
  return FUTX_OK;
}

futx_status futx_pack_fp8_weights_host(const futx_dims* dims, futx_proj proj, const float* w_host,
                                       const float* gain_host, void* packed_host, void* scales_host) {
  clear_error();
  ProjShape ps;
  futx_status st = fp8_shape(dims, proj, &ps);
  if (st) return st;
  if (!w_host || !packed_host || !scales_host) return fail(FUTX_E_ARG, "pack_fp8: null pointer");
  const int tiles = ps.n / 16;
  unsigned hw = std::thread::hardware_concurrency();
  int nthreads = (int)std::min<unsigned>(hw ? hw : 1, 32);
  if ((size_t)ps.n * ps.k < (1u << 20)) nthreads = 1;
  std::atomic<int> next{0};
  auto worker = [&]() {
    for (;;) {
      const int t = next.fetch_add(1);
      if (t >= tiles) return;
      fp8_pack_rows(w_host, gain_host, ps.k, t * 16, (t + 1) * 16, (uint8_t*)packed_host, (float*)scales_host);
    }
  };
  std::vector<std::thread> pool;
  for (int i = 1; i < nthreads; ++i) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
  return FUTX_OK;
}

futx_status futx_pack_fp8_weights(const futx_dims* dims, futx_proj proj, const float* w_host, const float* gain_host,
                                  void* packed_dev, void* scales_dev, void* stream) {
  clear_error();
  size_t pb, sb;
  futx_status st = futx_fp8_packed_sizes(dims, proj, &pb, &sb);
  if (st) return st;
  if (!packed_dev || !scales_dev) return fail(FUTX_E_ARG, "pack_fp8: null device pointer");
  std::vector<uint8_t> hp(pb), hs(sb);
  if ((st = futx_pack_fp8_weights_host(dims, proj, w_host, gain_host, hp.data(), hs.data()))) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if ((e = hipMemcpyAsync(packed_dev, hp.data(), pb, hipMemcpyHostToDevice, s)) != hipSuccess ||
      (e = hipMemcpyAsync(scales_dev, hs.data(), sb, hipMemcpyHostToDevice, s)) != hipSuccess ||
      (e = hipStreamSynchronize(s)) != hipSuccess)
    return fail(FUTX_E_HIP, "pack_fp8: %s", hipGetErrorString(e));
  return FUTX_OK;
}

futx_status futx_fp8_linear_workspace_size(const futx_dims* dims, futx_proj proj, int32_t max_batch, size_t* bytes) {
  clear_error();
  ProjShape ps;
  futx_status st = fp8_shape(dims, proj, &ps);
  if (st) return st;
  if (max_batch < 1 || max_batch > kMaxBatch || !bytes) return fail(FUTX_E_ARG, "fp8 workspace: batch 1..32");
  size_t m = 0;
  for (int b = 1; b <= max_batch; ++b) {
    const size_t v = fp8_ws(ps.n, ps.k, b, nullptr).bytes;
    if (v > m) m = v;
  }
  *bytes = m;
  return FUTX_OK;
}

futx_status futx_fp8_quantize_act(int32_t k, int32_t rows, const uint16_t* act, uint8_t* codes, float* scales,
                                  void* stream) {
  clear_error();
  if (k < kFp8Group || k % kFp8Group || k / kFp8Group > 65535 || rows < 1 || rows > 65535)
    return fail(FUTX_E_ARG, "fp8_quantize_act: k a positive multiple of 128, rows 1..65535");
  if (!act || !codes || !scales) return fail(FUTX_E_ARG, "fp8_quantize_act: null pointer");
  fp8_quant_act_kernel<<<dim3(k / kFp8Group, rows), 64, 0, (hipStream_t)stream>>>(act, k, codes, scales);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FUTX_E_HIP, "fp8_quantize_act: %s", hipGetErrorString(e));
  return FUTX_OK;
}

futx_status futx_fp8_linear(const futx_dims* dims, futx_proj proj, const futx_qweight* w, int32_t batch,
                            const uint16_t* act, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  ProjShape ps;
  futx_status st = fp8_shape(dims, proj, &ps);
  if (st) return st;
  if (!w || !w->packed || !w->scales || ((uintptr_t)w->packed & 15))
    return fail(FUTX_E_ARG, "fp8_linear: weights must be non-null and 16-byte aligned");
  if (batch < 1 || batch > kMaxBatch || !act || !out || !workspace)
    return fail(FUTX_E_ARG, "fp8_linear: bad arguments");
  const Fp8Ws ws = fp8_ws(ps.n, ps.k, batch, (char*)workspace);
  if (ws.bytes > workspace_bytes)
    return fail(FUTX_E_WORKSPACE, "fp8_linear: workspace %zu < %zu bytes", workspace_bytes, ws.bytes);
  hipStream_t s = (hipStream_t)stream;
  if ((st = futx_fp8_quantize_act(ps.k, batch, act, ws.codes, ws.scales, stream))) return st;
  hipError_t e;
  const Fp8Plan p = fp8_plan(ps.n, ps.k, batch);
  Fp8Args a{};
  a.w = (const uint4*)w->packed;
  a.sw = (const float*)w->scales;
  a.act = ws.codes;
  a.sa = ws.scales;
  a.out = p.splits > 1 ? ws.part : out;
  a.N = ps.n;
  a.K = ps.k;
  a.B = batch;
  a.kb_per_split = p.kb_per_split;
  a.items = p.items;
  a.wgs_per_split = p.wgs_per_split;
  auto k1 = fp8_gemm_kernel<1>, k2 = fp8_gemm_kernel<2>;
  auto k = batch <= 16 ? k1 : k2;
  if (p.lds > 64 * 1024 && (e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)p.lds)) != hipSuccess)
    return fail(FUTX_E_HIP, "fp8_linear: %s", hipGetErrorString(e));
  k<<<p.splits * p.wgs_per_split, 256, p.lds, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return fail(FUTX_E_HIP, "fp8_linear: gemm: %s", hipGetErrorString(e));
  if (p.splits > 1 && (e = launch_reduce(ws.part, p.splits, batch, ps.n, nullptr, nullptr, out, 0, s)) != hipSuccess)
    return fail(FUTX_E_HIP, "fp8_linear: reduce: %s", hipGetErrorString(e));
  return FUTX_OK;
}

}  // extern "C"
