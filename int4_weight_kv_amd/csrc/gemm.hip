// INT4 projection GEMM for decode (batch 1..32) on gfx950, with fused
// RMSNorm, residual and SwiGLU epilogues.
//
// The pages' decode path multiplies the activations with INT4 weights
// whose nibbles are turned into matrix-core operands in registers, without
// an intermediate tile in memory (FuTransformer abstract, airebao.com item
// page; kongchang.com/en, section "INT4 Decode: letting dequantization feed
// directly into MMA operands"), and folds the fixed RMSNorm gain into those
// weights (same article, section "FP8 Prefill: fusing GEMM and epilogue all
// the way").
//
// Work decomposition.  A workgroup owns a run of items (16-row weight
// tiles; for the SwiGLU projection gate/up tile pairs) over one K range.  It
// first stages that K range of the activation (all batch rows) in LDS as
// bf16 matrix-core operands (an fp32 source is rounded to bf16 there, which
// is the RMSNorm operand rounding), together with the exact (fp64) sum of
// those operands per weight group, which removes the nibble offset, and for
// an fp32 source the RMSNorm sum of squares.  Then each of its four waves
// streams its quarter of the K range of item after item: 128-bit loads, 16
// bytes per lane per 1 KB tile, in chunks of eight tiles with the next
// chunk always in flight, across item boundaries.  At the end of an item the
// four quarter sums are added in LDS and one wave (rotating) applies the
// epilogue while the others keep streaming.
#include "device.h"
#include "gemm.h"

namespace futx {

template <int G, int NF, int NT, bool F32, int EPI, int PAIR>
__global__ __launch_bounds__(256) void int4_gemm_kernel(GemmArgs a) {
  constexpr int NTW = PAIR ? 2 : 1;   // weight tiles per item (gate + up)
  constexpr int CHK = PAIR ? 4 : 8;   // K blocks per chunk and wave
  extern __shared__ __align__(16) uint8_t s_dyn[];
  // LDS: activation range [NT][B][row] bf16 | group sums [B][ngr] float2 |
  //      partials [2][4][NTW][NF][4][64] float | ss [B] float
  const int tid = threadIdx.x, lane = tid & 63, wq = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int B = a.B;
  const int KB = a.K >> 7;
  const int split = blockIdx.x / a.wgs_per_split, wj = blockIdx.x - split * a.wgs_per_split;
  const int kb0 = split * a.kb_per_wg, kb1 = min(kb0 + a.kb_per_wg, KB);
  const int krange = kb1 - kb0;
  const int it0 = (int)((long)wj * a.items / a.wgs_per_split);
  const int it1 = (int)((long)(wj + 1) * a.items / a.wgs_per_split);
  const int row = krange * 128 + 8;  // bf16 elements per LDS row (16 B pad)
  const int ngr = krange * 128 / G;
  uint16_t* const s_act = (uint16_t*)s_dyn;
  float2* const s_gsum = (float2*)(s_dyn + (size_t)NT * B * row * 2);
  float* const s_part = (float*)(s_gsum + (size_t)B * ngr);
  float* const s_ss = s_part + 2 * 4 * NTW * NF * 4 * 64;
  const int ngroups = a.K / G;

  // this wave's quarter of the K range, in chunks of CHK K blocks
  const int kbq = (krange + 3) / 4;
  const int q0 = min(kb0 + wq * kbq, kb1), q1 = min(q0 + kbq, kb1);
  const int cpi = (kbq + CHK - 1) / CHK;  // chunks per item (same for every wave)
  const int nchunks = (it1 - it0) * cpi;

  uint4 wA[CHK][NTW], wB[CHK][NTW];
  uint32_t sA[CHK][NTW][128 / G], sB[CHK][NTW][128 / G];
  // Loads are unconditional (out-of-range K blocks re-read the quarter's
  // first block and are not used) and scales stay raw bits until use, so
  // a wave never waits on one chunk while loading the next.
  auto load_chunk = [&](uint4 (&w)[CHK][NTW], uint32_t (&sc)[CHK][NTW][128 / G], int c) {
    const int item = it0 + c / cpi, cb = q0 + (c % cpi) * CHK;
#pragma unroll
    for (int i = 0; i < CHK; ++i) {
      const int kb = cb + i < q1 ? cb + i : (q0 < q1 ? q0 : kb0);
#pragma unroll
      for (int u = 0; u < NTW; ++u) {
        const int nt = PAIR ? 2 * item + u : item;
        w[i][u] = a.w[((size_t)nt * KB + kb) * 64 + lane];
#pragma unroll
        for (int gi = 0; gi < 128 / G; ++gi)
          sc[i][u][gi] = a.sc[(size_t)(nt * 16 + col) * ngroups + kb * (128 / G) + gi];
      }
    }
  };
  if (nchunks > 0) load_chunk(wA, sA, 0);
  if (nchunks > 1) load_chunk(wB, sB, 1);

  // ---- stage the activation range once: bf16 operands, exact group sums,
  // RMSNorm sum of squares (deterministic order)
  {
    const int c8 = krange * 16;  // 8-element chunks per row
    const int total = B * c8;
    for (int it = 0; it * 256 < total; ++it) {
      const int idx = it * 256 + tid;
      const bool ok = idx < total;
      const int b = ok ? idx / c8 : 0, k8 = ok ? idx - b * c8 : 0;
      double gs = 0.0;
      float sq = 0.f;
      if (ok) {
        const size_t src = (size_t)b * a.K + kb0 * 128 + k8 * 8;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          uint4 v;
          if constexpr (F32) {
            const float4* q = (const float4*)((const float*)a.act + src);
            const float4 x0 = q[0], x1 = q[1];
            v = uint4{pack2_bf16(x0.x, x0.y), pack2_bf16(x0.z, x0.w), pack2_bf16(x1.x, x1.y), pack2_bf16(x1.z, x1.w)};
            sq = fmaf(x0.x, x0.x, fmaf(x0.y, x0.y, fmaf(x0.z, x0.z, fmaf(x0.w, x0.w, sq))));
            sq = fmaf(x1.x, x1.x, fmaf(x1.y, x1.y, fmaf(x1.z, x1.z, fmaf(x1.w, x1.w, sq))));
          } else {
            v = *(const uint4*)((const uint16_t*)a.act + t * a.term_stride + src);
          }
          *(uint4*)(s_act + (size_t)(t * B + b) * row + k8 * 8) = v;
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int c = 0; c < 4; ++c)
            gs += (double)bf16_bits_to_f32(w4[c] & 0xFFFF) + (double)bf16_bits_to_f32(w4[c] >> 16);
        }
      }
      // a weight group is G / 8 consecutive chunks = consecutive lanes
#pragma unroll
      for (int o = 1; o < G / 8; o <<= 1) {
        gs += __shfl_xor(gs, o, 64);
        if constexpr (F32) sq += __shfl_xor(sq, o, 64);
      }
      if (ok && (k8 % (G / 8)) == 0) {
        s_gsum[(size_t)b * ngr + k8 / (G / 8)] = split_f64(gs);
        if constexpr (F32) s_part[(size_t)b * ngr + k8 / (G / 8)] = sq;  // scratch until the loop
      }
    }
    __syncthreads();
    if constexpr (F32) {
      if (tid < B) {
        float t = 0.f;
        for (int g = 0; g < ngr; ++g) t += s_part[(size_t)tid * ngr + g];
        s_ss[tid] = t;
      }
      __syncthreads();
    }
  }

  // ---- stream: chunk c of item it0 + c / cpi
  f32x4 acc[NTW][NF];
  auto zero_acc = [&]() {
#pragma unroll
    for (int u = 0; u < NTW; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[u][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  zero_acc();

  auto compute = [&](const uint4 (&w)[CHK][NTW], const uint32_t (&sc)[CHK][NTW][128 / G], int c) {
    const int cb = q0 + (c % cpi) * CHK;
#pragma unroll
    for (int i = 0; i < CHK; ++i) {
      const int kb = cb + i;
      if (kb < q1) {
        const int kl = (kb - kb0) * 128;
#pragma unroll
        for (int gi = 0; gi < 128 / G; ++gi) {
          f32x4 d[NTW][NF];
#pragma unroll
          for (int u = 0; u < NTW; ++u)
#pragma unroll
            for (int f = 0; f < NF; ++f) d[u][f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ss = 0; ss < G / 32; ++ss) {
            const int s = gi * (G / 32) + ss;
            bf16x8 bw[NTW];
#pragma unroll
            for (int u = 0; u < NTW; ++u) bw[u] = widen_word(word_of(w[i][u], s));
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
              for (int f = 0; f < NF; ++f) {
                const int tok = f * 16 + col;
                uint4 v = {0u, 0u, 0u, 0u};
                if (tok < B) v = *(const uint4*)(s_act + (size_t)(t * B + tok) * row + kl + s * 32 + grp * 8);
                const bf16x8 av = as_bf16x8(v);
#pragma unroll
                for (int u = 0; u < NTW; ++u) d[u][f] = mfma16(av, bw[u], d[u][f]);
              }
          }
          const int jl = kl / G + gi;
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int tok = f * 16 + 4 * grp + r;
              const float2 gs = tok < B ? s_gsum[(size_t)tok * ngr + jl] : float2{0.f, 0.f};
#pragma unroll
              for (int u = 0; u < NTW; ++u)
                acc[u][f][r] = fmaf(half_bits_to_f32((uint16_t)sc[i][u][gi]), remove_offset(d[u][f][r], gs), acc[u][f][r]);
            }
        }
      }
    }
  };

  auto part = [&](int slot, int w, int u, int f, int r) -> float& {
    return s_part[((((slot * 4 + w) * NTW + u) * NF + f) * 4 + r) * 64 + lane];
  };

  // end of an item: add the four quarters in LDS; one wave (rotating)
  // applies the epilogue while the others go on streaming
  auto finish_item = [&](int item, int slot) {
#pragma unroll
    for (int u = 0; u < NTW; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r) part(slot, wq, u, f, r) = acc[u][f][r];
    zero_acc();
    __syncthreads();
    if (wq != ((item - it0) & 3)) return;
    float o[NTW][NF][4];
#pragma unroll
    for (int u = 0; u < NTW; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o[u][f][r] = (part(slot, 0, u, f, r) + part(slot, 1, u, f, r)) + (part(slot, 2, u, f, r) + part(slot, 3, u, f, r));
    const int n = item * 16 + col;  // physical row (non-pair) / logical column (pair)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = f * 16 + 4 * grp + r;
        if (tok >= B) continue;
        if constexpr (EPI == kEpiPartial) {
          a.out[((size_t)split * B + tok) * a.N + n] = o[0][f][r];
        } else if constexpr (EPI == kEpiRms) {
          a.out[(size_t)tok * a.N + n] = o[0][f][r] * (1.0f / sqrtf(s_ss[tok] / (float)a.K + a.eps));
        } else if constexpr (EPI == kEpiResid) {
          a.out[(size_t)tok * a.N + n] = a.resid[(size_t)tok * a.N + n] + o[0][f][r];
        } else {  // kEpiSwiglu: u = 0 gate rows, u = 1 up rows of logical column n
          const float invr = 1.0f / sqrtf(s_ss[tok] / (float)a.K + a.eps);
          const float g = o[0][f][r] * invr, up = o[PAIR][f][r] * invr;
          a.out_bf16[(size_t)tok * a.inter + n] = f32_to_bf16_bits(g / (1.0f + expf(-g)) * up);
        }
      }
  };

  for (int c = 0; c < nchunks; c += 2) {
    compute(wA, sA, c);
    if (c + 2 < nchunks) load_chunk(wA, sA, c + 2);
    if ((c + 1) % cpi == 0) finish_item(it0 + c / cpi, (c / cpi) & 1);
    if (c + 1 < nchunks) {
      compute(wB, sB, c + 1);
      if (c + 3 < nchunks) load_chunk(wB, sB, c + 3);
      if ((c + 2) % cpi == 0) finish_item(it0 + (c + 1) / cpi, ((c + 1) / cpi) & 1);
    }
  }
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

size_t gemm_lds_bytes(const GemmArgs& a, int nterms, int G, bool pair) {
  const int krange = a.kb_per_wg;
  const int nf = a.B <= 16 ? 1 : 2;
  const size_t act = (size_t)nterms * a.B * ((size_t)krange * 128 + 8) * 2;
  const size_t gs = (size_t)a.B * (krange * 128 / G) * 8;
  const size_t prt = (size_t)2 * 4 * (pair ? 2 : 1) * nf * 4 * 64 * 4;
  const size_t sq = (size_t)a.B * (krange * 128 / G) * 4;  // scratch, aliases the partials
  return act + gs + (prt > sq ? prt : sq) + (size_t)a.B * 4;
}

GemmPlan2 plan_gemm(int N, int K, int G, int B, int nterms, int epi) {
  GemmPlan2 p;
  const int KB = K / 128;
  const int items = epi == kEpiSwiglu ? N / 32 : N / 16;
  // K splits: only kEpiPartial may split; split until the activation range
  // fits the LDS budget
  p.splits = 1;
  if (epi == kEpiPartial) {
    while (p.splits < KB && (long)nterms * B * ((KB + p.splits - 1) / p.splits) * 256 > kLdsActBudget) ++p.splits;
  }
  p.kb_per_wg = (KB + p.splits - 1) / p.splits;
  p.splits = (KB + p.kb_per_wg - 1) / p.kb_per_wg;
  // workgroups per split: about two per CU in total
  const int cus = device_cu_count();
  int w = (2 * cus + p.splits - 1) / p.splits;
  p.wgs_per_split = w < items ? w : items;
  p.items = items;
  return p;
}

bool gemm_fits(int K, int G, int B, int nterms, int epi) {
  GemmArgs a{};
  a.B = B;
  const GemmPlan2 p = plan_gemm(16, K, G, B, nterms, epi);
  a.kb_per_wg = p.kb_per_wg;
  return gemm_lds_bytes(a, nterms, G, epi == kEpiSwiglu) <= kLdsMax;
}

hipError_t launch_int4_gemm(GemmArgs a, int G, int nterms, bool act_f32, int epi, hipStream_t st) {
  const bool pair = epi == kEpiSwiglu;
  const dim3 grid(a.splits * a.wgs_per_split), block(256);
  if (a.splits != 1 && epi != kEpiPartial) return hipErrorInvalidValue;
  const size_t lds = gemm_lds_bytes(a, nterms, G, pair);
  if (lds > (size_t)kLdsMax) return hipErrorInvalidValue;
#define FUTX_G(GG, NF, NT, F32, EPI, PR) \
  do {                                   \
    auto k_ = int4_gemm_kernel<GG, NF, NT, F32, EPI, PR>; \
    if (lds > 64 * 1024) hipFuncSetAttribute((const void*)k_, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    k_<<<grid, block, lds, st>>>(a); \
  } while (0)
#define FUTX_NF(GG, NT, F32, EPI, PR) \
  do {                                  \
    if (a.B <= 16) FUTX_G(GG, 1, NT, F32, EPI, PR); else FUTX_G(GG, 2, NT, F32, EPI, PR); \
  } while (0)
#define FUTX_GRP(NT, F32, EPI, PR)                                        \
  do {                                                                     \
    if (G == 128) FUTX_NF(128, NT, F32, EPI, PR); else FUTX_NF(64, NT, F32, EPI, PR); \
  } while (0)
  switch (epi) {
    case kEpiPartial:
      if (nterms == 3) FUTX_GRP(3, false, kEpiPartial, 0);
      else if (act_f32) FUTX_GRP(1, true, kEpiPartial, 0);
      else FUTX_GRP(1, false, kEpiPartial, 0);
      break;
    case kEpiRms: FUTX_GRP(1, true, kEpiRms, 0); break;
    case kEpiResid:
      if (nterms == 3) FUTX_GRP(3, false, kEpiResid, 0); else FUTX_GRP(1, false, kEpiResid, 0);
      break;
    case kEpiSwiglu: FUTX_GRP(1, true, kEpiSwiglu, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef FUTX_GRP
#undef FUTX_NF
#undef FUTX_G
  return hipGetLastError();
}

}  // namespace futx
