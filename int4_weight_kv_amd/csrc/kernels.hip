// gfx950 kernels of the INT4 decode block (multi-kernel path).
//
// Each kernel implements one step of the decode block described in the
// FuTransformer abstract (airebao.com item page) and the kongchang.com/en
// article, section "INT4 Decode: letting dequantization feed directly into
// MMA operands": INT4 projections whose nibbles are widened to bf16 in
// registers and fed to the matrix cores, a rotated INT4 KV cache, and
// split-sequence decode attention.  Operand and cache layouts: layout.h.
#include <cmath>

#include "device.h"
#include "gemm.h"
#include "futx.h"
#include "kernels.h"

namespace futx {

// ---------------------------------------------------------------- activations

// invr[b] = 1 / sqrt(mean(x[b]^2) + eps); act[b][:] = bf16(x[b][:]) when act
// is not null.
// RMSNorm reading: the gain lives in the next weights and 1/r is applied to
// the GEMM result, so the matrix-core operand is bf16(x).
__global__ __launch_bounds__(1024) void prep_act_kernel(const float* __restrict__ x, int H, float eps,
                                                        uint16_t* __restrict__ act,
                                                        float* __restrict__ invr) {
  // one 1024-thread workgroup per row, 16-byte loads (H is a multiple of
  // 128), all of a thread's loads issued before the first use
  const int b = blockIdx.x;
  const float4* xr = (const float4*)(x + (size_t)b * H);
  const int n4 = H >> 2;
  float ss = 0.f;
#pragma unroll 4
  for (int i = threadIdx.x; i < n4; i += 1024) {
    const float4 v = xr[i];
    ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
    if (act) {
      uint2 o;
      o.x = f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
      o.y = f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16);
      ((uint2*)(act + (size_t)b * H))[i] = o;
    }
  }
  __shared__ float red[16];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < 16; ++w) t += red[w];
    invr[b] = 1.0f / sqrtf(t / (float)H + eps);
  }
}

// ---------------------------------------------------- split-K epilogues
// (the INT4 GEMM itself is in gemm.hip; with K split it writes fp32 partial
// sums part[split][b][P] in physical row order, finished here)

// logical row n of a projection output -> physical row (GATEUP tiles
// alternate gate / up; identity otherwise)
__device__ __forceinline__ int physical_row(int n, int gateup_inter) {
  if (!gateup_inter) return n;
  const int half = n / gateup_inter, r = n - half * gateup_inter;
  return (2 * (r >> 4) + half) * 16 + (r & 15);
}

__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ part, int S, int B,
                                                     int N, const float* __restrict__ rowscale,
                                                     const float* resid, float* out,
                                                     int gateup_inter) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= B * N) return;
  const int b = idx / N, n = idx - b * N;
  const int P = physical_row(n, gateup_inter);
  // partials summed in split order; up to 8 loads in flight per round trip
  float s = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = s0 + j < S ? part[((size_t)(s0 + j) * B + b) * N + P] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) s += v[j];
  }
  if (rowscale) s *= rowscale[b];
  if (resid) s += resid[idx];
  out[idx] = s;
}

// SwiGLU of the gate/up partials: act[b][c] = bf16(silu(g) * u) with
// g = invr[b] * sum(gate partials), u = invr[b] * sum(up partials).
__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ part, int S, int B, int I,
                                                     const float* __restrict__ invr, uint16_t* __restrict__ act) {
  const int c = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  if (c >= I) return;
  const int N = 2 * I;
  const int Pg = 32 * (c >> 4) + (c & 15), Pu = Pg + 16;
  // partials summed in split order; up to 8 splits in flight per round trip
  float g = 0.f, u = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float vg[8], vu[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const size_t o = ((size_t)(s0 + j) * B + b) * N;
      vg[j] = s0 + j < S ? part[o + Pg] : 0.f;
      vu[j] = s0 + j < S ? part[o + Pu] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) {
        g += vg[j];
        u += vu[j];
      }
  }
  g *= invr[b];
  u *= invr[b];
  act[(size_t)b * I + c] = f32_to_bf16_bits(g / (1.0f + expf(-g)) * u);
}

// ---------------------------------------------------------------- KV append

// cos / sin of the RoPE angle pos * theta^(-2i/d).  The angle is formed and
// reduced modulo 2 pi in fp64 (Cody-Waite with a two-part 2 pi), so long
// positions keep full accuracy; fp64 sin / cos of the reduced angle in
// [-pi, pi] then cost no large-argument reduction, and the fp32 results are
// the correctly rounded values but for rare double-rounding cases.
__device__ __forceinline__ void rope_cs_inv(int pos, double inv, float* c, float* s) {
  const double ang = (double)pos * inv;
  constexpr double kTwoPiHi = 6.28318530717958623200e+00;  // 2 pi rounded to double
  constexpr double kTwoPiLo = 2.44929359829470635445e-16;  // 2 pi - kTwoPiHi
  const double k = rint(ang * (1.0 / kTwoPiHi));
  const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));
  double sn, cs;
  sincos(r, &sn, &cs);  // |r| <= pi: no large-argument reduction left
  *s = (float)sn;
  *c = (float)cs;
}

__device__ __forceinline__ void rope_cs(int pos, int i, int d, float theta, float* c, float* s) {
  rope_cs_inv(pos, exp2(-2.0 * (double)i / (double)d * log2((double)theta)), c, s);
}

// Rotate-half RoPE of one head held as channel c = lane + 64 j, given cos /
// sin of frequency index lane % (D / 2) (rope_cs).
template <int D>
__device__ __forceinline__ void rope_lane_cs(float (&x)[D / 64], float c, float s) {
  const int lane = threadIdx.x & 63;
  if constexpr (D == 128) {
    const float a = x[0], b = x[1];
    x[0] = a * c - b * s;
    x[1] = b * c + a * s;
  } else {
    const float o = __shfl_xor(x[0], 32, 64);
    x[0] = lane < 32 ? x[0] * c - o * s : x[0] * c + o * s;
  }
}

template <int D>
__device__ __forceinline__ void rope_lane(float (&x)[D / 64], int pos, float theta) {
  float c, s;
  rope_cs(pos, (threadIdx.x & 63) % (D / 2), D, theta, &c, &s);
  rope_lane_cs<D>(x, c, s);
}

// Normalized Sylvester Hadamard over contiguous blocks of hb channels
// (hb divides 64, so a block never leaves its 64-lane row).
template <int HOP, int D>
__device__ __forceinline__ void fwht_hop(float (&x)[D / 64]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    float o;
    if constexpr (HOP >= 16) o = xor_lanes<HOP>(x[j]);
    else o = __shfl_xor(x[j], HOP, 64);
    x[j] = (lane & HOP) ? o - x[j] : x[j] + o;
  }
}

template <int D>
__device__ __forceinline__ void fwht_lane(float (&x)[D / 64], int hb) {
  if (hb > 1) fwht_hop<1, D>(x);
  if (hb > 2) fwht_hop<2, D>(x);
  if (hb > 4) fwht_hop<4, D>(x);
  if (hb > 8) fwht_hop<8, D>(x);
  if (hb > 16) fwht_hop<16, D>(x);
  if (hb > 32) fwht_hop<32, D>(x);
  const float sc = 1.0f / sqrtf((float)hb);
#pragma unroll
  for (int j = 0; j < D / 64; ++j) x[j] *= sc;
}

// Per-(token, head) INT4 quantization (fp32 recipe, scale saturated at the
// fp16 maximum).  Returns the fp16 scale bits; codes in q[].
template <int D>
__device__ __forceinline__ uint16_t quantize_lane(const float (&x)[D / 64], int (&q)[D / 64]) {
  float am = 0.f;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) am = fmaxf(am, fabsf(x[j]));
  am = wave_max(am);
  const float s32 = fminf(am / 7.0f, 65504.0f);
  const __half s16 = __float2half_rn(s32);
  const float sf = __half2float(s16);
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    float v = sf == 0.f ? 0.f : rintf(x[j] / sf);
    q[j] = (int)fminf(fmaxf(v, -8.f), 7.f);
  }
  return __half_as_ushort(s16);
}

// One new token of KV head h in registers: the codes of channel
// c = lane + 64 j (quantize_lane), the packed key word of the lane's run of
// 8 channels (valid in lanes with lane % 8 == 0, channels lane + 64 j ..
// lane + 64 j + 7, in the key layout of layout.h) and the fp16 scales.
template <int D>
struct TokenCodes {
  int qk[D / 64], qv[D / 64];
  uint32_t kword[D / 64];
  uint16_t sk, sv;
};

template <int D>
__device__ __forceinline__ void quantize_token(const float (&kx)[D / 64], const float (&vx)[D / 64],
                                               TokenCodes<D>& t) {
  const int lane = threadIdx.x & 63, e = lane & 7;
  t.sk = quantize_lane<D>(kx, t.qk);
  t.sv = quantize_lane<D>(vx, t.qv);
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    uint32_t w = nibble_bits(e, (uint32_t)(t.qk[j] + (int)kNibbleBias));
    w |= __shfl_xor(w, 1, 64);
    w |= __shfl_xor(w, 2, 64);
    w |= __shfl_xor(w, 4, 64);
    t.kword[j] = w;
  }
}

// Writes one quantized token of KV head h into its slot.
template <int D>
__device__ void store_token(const TokenCodes<D>& t, int slot, int h, const KVPtrs& kv) {
  const int lane = threadIdx.x & 63;
  const int page = slot / kPageSize, off = slot % kPageSize;
  const size_t head_base = ((size_t)page * kv.nkv + h) * (size_t)(kPageSize * D / 2);
  // keys: the word of 8 consecutive channels of token off
  const int e = lane & 7, g = (lane & 31) >> 3;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    if (e == 0) {
      const int s = (lane >> 5) + 2 * j;
      uint8_t* p = kv.k_codes + head_base + (size_t)(off >> 4) * (8 * D) +
                   (size_t)(g * 16 + (off & 15)) * (D / 8) + s * 4;
      *(uint32_t*)p = t.kword[j];
    }
  }
  // values: one nibble per channel in a word shared with 7 other tokens
  const int tb = off >> 5, tp = off & 31;
  const int gv = tp < 16 ? tp >> 2 : (tp - 16) >> 2;
  const int ev = tp < 16 ? (tp & 3) : 4 + ((tp - 16) & 3);
  const uint32_t vmask = nibble_bits(ev, 15u);
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    const int c = lane + 64 * j;
    const int cg = c >> 6, c4 = (c & 63) >> 4;
    uint32_t* p = (uint32_t*)(kv.v_codes + head_base + (size_t)(tb * (D / 64) + cg) * 1024 +
                              (size_t)(gv * 16 + (c & 15)) * 16 + c4 * 4);
    atomicAnd(p, ~vmask);
    atomicOr(p, nibble_bits(ev, (uint32_t)(t.qv[j] + (int)kNibbleBias)));
  }
  if (lane == 0) {
    kv.k_scales[((size_t)page * kv.nkv + h) * kPageSize + off] = t.sk;
    kv.v_scales[((size_t)page * kv.nkv + h) * kPageSize + off] = t.sv;
  }
}

template <int D>
__global__ __launch_bounds__(64) void kv_append_kernel(const float* __restrict__ k,
                                                       const float* __restrict__ v,
                                                       const int32_t* __restrict__ positions,
                                                       const int32_t* __restrict__ slots,
                                                       uint32_t flags, int hb, float theta,
                                                       KVPtrs kv) {
  const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const size_t base = ((size_t)t * kv.nkv + h) * D;
  float kx[D / 64], vx[D / 64];
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    kx[j] = k[base + lane + 64 * j];
    vx[j] = v[base + lane + 64 * j];
  }
  if (flags & FUTX_KV_ROPE) rope_lane<D>(kx, positions[t], theta);
  if (flags & FUTX_KV_HADAMARD) {
    fwht_lane<D>(kx, hb);
    fwht_lane<D>(vx, hb);
  }
  TokenCodes<D> tc;
  quantize_token<D>(kx, vx, tc);
  store_token<D>(tc, slots[t], h, kv);
}

// ---------------------------------------------------------------- attention

// Split-sequence decode attention.  One wave per (chunk, KV head, sequence)
// computes, for the G query heads of the KV head, the chunk's running max m,
// normalizer l and unnormalized p.v accumulator over rotated INT4 keys and
// values (flash-decoding partials, merged as attn_decode_kernel describes).
//   q.k:  A = key tile (16 tokens x 32 channels per MFMA), B = rotated query
//         (query heads as columns) -> scores[token][head] with the token of
//         lane L, reg r at 4 (L/16) + r.
//   p.v:  A = probabilities (heads x 32 tokens) built directly from the two
//         score tiles of a 32-token block, B = value tile.
// Precision: the attention output feeds a bf16 rounding point (the O
// projection operand), so it is kept at fp32 accuracy.  Keys and values
// widen to their exact signed codes in fp16 (no offset term in the fp32
// accumulators), and the two fp32 operands (query, p * value scale) enter
// the fp16 MFMA as a hi + lo pair (22 significant bits) after an exact
// power-of-two scaling into fp16 range.
__device__ __forceinline__ uint32_t pack_h2(_Float16 a, _Float16 b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// x (already scaled into fp16 range) -> fp16 hi + lo
__device__ __forceinline__ void split_f16(float x, _Float16* hi, _Float16* lo) {
  *hi = (_Float16)x;
  *lo = (_Float16)(x - (float)*hi);
}

// Scores are kept in base-2 units (the query scale carries log2 e), so the
// softmax weights are single exp2 evaluations: exp(x) = 2^(x log2 e).
constexpr float kLog2e = 1.44269504088896340736f;

// power-of-two exponent k such that m * 2^k lies in [2^(top-1), 2^top)
__device__ __forceinline__ int range_exp(float m, int top) {
  if (!(m > 0.f)) return 0;
  int e;
  (void)frexpf(m, &e);  // m = f * 2^e, f in [0.5, 1)
  return top - e;
}

// A 32-token block of one page and KV head in the attention operand layout
// (layout.h): key words of its two 16-token tiles, value words of its
// channel groups, and the fp16 scales of the tokens 4 grp + r of each tile.
template <int D>
struct KvBlk {
  uint32_t kw[2][D / 32];
  uint4 vw[D / 64];
  uint2 k2[2], v2[2];
};

template <int D>
__device__ __forceinline__ void load_blk(const KVPtrsConst& kv, int page, int off, int h, KvBlk<D>& r) {
  const int lane = threadIdx.x & 63, grp = lane >> 4;
  const size_t hb_off = ((size_t)page * kv.nkv + h) * ((size_t)kPageSize * D / 2);
  const size_t sc_off = ((size_t)page * kv.nkv + h) * kPageSize + off;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint8_t* p = kv.k_codes + hb_off + (size_t)((off >> 4) + u) * (8 * D) + (size_t)lane * (D / 8);
    if constexpr (D == 128) {
      const uint4 v = *(const uint4*)p;
      r.kw[u][0] = v.x; r.kw[u][1] = v.y; r.kw[u][2] = v.z; r.kw[u][3] = v.w;
    } else {
      const uint2 v = *(const uint2*)p;
      r.kw[u][0] = v.x; r.kw[u][1] = v.y;
    }
  }
#pragma unroll
  for (int cg = 0; cg < D / 64; ++cg)
    r.vw[cg] = *(const uint4*)(kv.v_codes + hb_off + (size_t)((off >> 5) * (D / 64) + cg) * 1024 + (size_t)lane * 16);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    r.k2[u] = *(const uint2*)(kv.k_scales + sc_off + 16 * u + 4 * grp);
    r.v2[u] = *(const uint2*)(kv.v_scales + sc_off + 16 * u + 4 * grp);
  }
}

// The new token as a block whose token 0 it is (tokens 1..31 are masked by
// the caller's length).  Key word s of lane L (token L % 16, channels
// 32 s + 8 (L / 16) + e) is the packed word of lane 8 (L / 16) + 32 (s % 2),
// run s / 2; value word c4 of channel group cg holds the code of channel
// cg * 64 + 16 c4 + L % 16 in element 0 (token 0) and code 0 elsewhere.
// The codes are the ones written to the cache, so the token enters exactly
// as it would when read back.
template <int D>
__device__ __forceinline__ void token_blk(const TokenCodes<D>& t, KvBlk<D>& r) {
  const int lane = threadIdx.x & 63, grp = lane >> 4;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const uint32_t w = __shfl(t.kword[s >> 1], 8 * grp + 32 * (s & 1), 64);
    r.kw[0][s] = w;
    r.kw[1][s] = w;
  }
  uint32_t zero_codes = 0;
#pragma unroll
  for (int e = 1; e < 8; ++e) zero_codes |= nibble_bits(e, kNibbleBias);
#pragma unroll
  for (int cg = 0; cg < D / 64; ++cg) {
    uint32_t w4[4];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int code = __shfl(t.qv[cg], 16 * c4 + (lane & 15), 64);
      w4[c4] = zero_codes | nibble_bits(0, (uint32_t)(code + (int)kNibbleBias));
    }
    r.vw[cg] = uint4{w4[0], w4[1], w4[2], w4[3]};
  }
  r.k2[0] = uint2{(uint32_t)t.sk, 0u};
  r.k2[1] = uint2{0u, 0u};
  r.v2[0] = uint2{(uint32_t)t.sv, 0u};
  r.v2[1] = uint2{0u, 0u};
}

// Online-softmax update with one 32-token block starting at token blk
// (tokens >= t1 masked; at least one token of the block must be < t1):
// running max m_i (base-2 score units) and normalizer part l_part of query
// head col (per lane),
// p.v accumulators acc (row 4 grp + r = head, column = channel).
template <int D>
__device__ __forceinline__ void compute_blk(int blk, int t1, const KvBlk<D>& rb, const f16x8 (&qh)[D / 32],
                                            const f16x8 (&ql)[D / 32], float zscale, float& m_i, float& l_part,
                                            f32x4 (&acc)[D / 16]) {
  const int lane = threadIdx.x & 63, grp = lane >> 4;
  const NibRegs nk = nib_regs_f16();
  float ks[2][4], vs[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint2 k2 = rb.k2[u], v2 = rb.v2[u];
    ks[u][0] = half_bits_to_f32(k2.x & 0xFFFF); ks[u][1] = half_bits_to_f32(k2.x >> 16);
    ks[u][2] = half_bits_to_f32(k2.y & 0xFFFF); ks[u][3] = half_bits_to_f32(k2.y >> 16);
    vs[u][0] = half_bits_to_f32(v2.x & 0xFFFF); vs[u][1] = half_bits_to_f32(v2.x >> 16);
    vs[u][2] = half_bits_to_f32(v2.y & 0xFFFF); vs[u][3] = half_bits_to_f32(v2.y >> 16);
  }
  // scores
  float z[2][4];
  float mloc = -INFINITY;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const f16x8 kc = widen_word_exact_f16(rb.kw[u][s], nk);
      d = mfma16h(kc, qh[s], d);
      d = mfma16h(kc, ql[s], d);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = blk + 16 * u + 4 * grp + r;
      z[u][r] = t < t1 ? d[r] * ks[u][r] * zscale : -INFINITY;
      if (t >= t1) vs[u][r] = 0.f;  // stale scales past the end stay out of p.v
      mloc = fmaxf(mloc, z[u][r]);
    }
  }
  mloc = fmaxf(mloc, xor_lanes<16>(mloc));
  mloc = fmaxf(mloc, xor_lanes<32>(mloc));
  const float m_new = fmaxf(m_i, mloc);
  const float alpha = __builtin_amdgcn_exp2f(m_i - m_new);
  // exact power-of-two scaling of p * vs (<= max vs) into fp16 range
  float vmax = fmaxf(fmaxf(fmaxf(vs[0][0], vs[0][1]), fmaxf(vs[0][2], vs[0][3])),
                     fmaxf(fmaxf(vs[1][0], vs[1][1]), fmaxf(vs[1][2], vs[1][3])));
  vmax = fmaxf(vmax, xor_lanes<16>(vmax));
  vmax = fmaxf(vmax, xor_lanes<32>(vmax));
  const int kp = range_exp(vmax, 14);
  float psum = 0.f;
  uint32_t phw[4], plw[4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int r = 0; r < 4; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(z[u][r] - m_new), p1 = __builtin_amdgcn_exp2f(z[u][r + 1] - m_new);
      psum += p0 + p1;
      _Float16 h0, l0, h1, l1;
      split_f16(ldexpf(p0 * vs[u][r], kp), &h0, &l0);
      split_f16(ldexpf(p1 * vs[u][r + 1], kp), &h1, &l1);
      phw[2 * u + r / 2] = pack_h2(h0, h1);
      plw[2 * u + r / 2] = pack_h2(l0, l1);
    }
  }
  l_part = l_part * alpha + psum;
  m_i = m_new;
  const f16x8 pah = __builtin_bit_cast(f16x8, u32x4{phw[0], phw[1], phw[2], phw[3]});
  const f16x8 pal = __builtin_bit_cast(f16x8, u32x4{plw[0], plw[1], plw[2], plw[3]});
  // rescale the p.v accumulators: row 4 (L/16) + r belongs to head 4 grp + r.
  // When no head of the wave moved its running max (alpha = 1 everywhere,
  // the usual case once the max has settled), the rescale is the identity:
  // the update fma(dv, pback, acc) is then the same number, and the row
  // factors are not gathered.
  const bool moved = __any(alpha != 1.0f);  // wave-uniform
  float al[4] = {1.f, 1.f, 1.f, 1.f};
  if (moved) {
#pragma unroll
    for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * grp + r, 64);
  }
  const float pback = ldexpf(1.0f, -kp);
#pragma unroll
  for (int cg = 0; cg < D / 64; ++cg)
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const f16x8 vc = widen_word_exact_f16(word_of(rb.vw[cg], c4), nk);
      f32x4 dv = mfma16h(pah, vc, f32x4{0.f, 0.f, 0.f, 0.f});
      dv = mfma16h(pal, vc, dv);
      if (moved) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[cg * 4 + c4][r] = fmaf(acc[cg * 4 + c4][r], al[r], dv[r] * pback);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[cg * 4 + c4][r] = fmaf(dv[r], pback, acc[cg * 4 + c4][r]);
      }
    }
}

// The two 32-token halves of cache page `pg` for KV head h.
template <int D>
__device__ __forceinline__ void issue_page(const KVPtrsConst& kv, int pg, int h, KvBlk<D>& r0, KvBlk<D>& r1) {
  load_blk<D>(kv, pg, 0, h, r0);
  load_blk<D>(kv, pg, 32, h, r1);
}

// Online-softmax scan of tokens [t0, t1) of one sequence (block table row
// bt, t0 page-aligned, page index pg0 = t0 / page size) against KV head h.
// btv holds the row's entries pg0 + j in lane j (j < 63; lane 63 holds the
// sequence's first page), so the page of a later step is read from a
// register, not from memory.  The caller issued the first page into a0 / a1
// and the second (or the first again) into b0 / b1.  Pages are
// double-buffered: after page i is computed, the loads of page i + 2 go into
// its registers; past the last page the loads repeat it (valid addresses)
// and are not used.
template <int D>
__device__ __forceinline__ void split_scan(const f16x8 (&qh)[D / 32], const f16x8 (&ql)[D / 32],
                                           const float& zscale, const int32_t* bt, int btv, int pg0, int t0,
                                           int t1, int h, const KVPtrsConst& kv, float& m_i, float& l_part,
                                           f32x4 (&acc)[D / 16], KvBlk<D>& a0, KvBlk<D>& a1, KvBlk<D>& b0,
                                           KvBlk<D>& b1) {
  auto issue = [&](int pt, KvBlk<D>& r0, KvBlk<D>& r1) {
    const int pi = min(pt, t1 - 1) / kPageSize;
    const int j = pi - pg0;  // uniform
    const int pg = j < 63 ? __builtin_amdgcn_readlane(btv, j) : bt[pi];
    issue_page<D>(kv, pg, h, r0, r1);
  };
  auto consume = [&](int pt, const KvBlk<D>& r0, const KvBlk<D>& r1) {
    compute_blk<D>(pt, t1, r0, qh, ql, zscale, m_i, l_part, acc);
    if (pt + 32 < t1) compute_blk<D>(pt + 32, t1, r1, qh, ql, zscale, m_i, l_part, acc);
  };
  int pt = t0;
  for (;;) {
    consume(pt, a0, a1);
    pt += kPageSize;
    if (pt >= t1) break;
    issue(pt + kPageSize, a0, a1);
    consume(pt, b0, b1);
    pt += kPageSize;
    if (pt >= t1) break;
    issue(pt + kPageSize, b0, b1);
  }
}

// o (fp32, channel c of query head i) -> the O projection operand: NT bf16
// terms, each the bf16 rounding of what the terms before it leave (two
// terms: 16 significant bits; three: 24), term t at out + t * stride.
template <int NT>
__device__ __forceinline__ void store_terms(float o, uint16_t* out, size_t at, size_t term_stride) {
  float r = o;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint16_t v = f32_to_bf16_bits(r);
    out[at + t * term_stride] = v;
    r -= bf16_bits_to_f32(v);
  }
}

// o (fp32) of query head channel c, held in lane c % 64 of a wave whose 64
// lanes hold 64 consecutive channels: the inverse block rotation (the
// normalized Sylvester matrix is its own inverse), then the output at
// element `at` (fp32, and / or FUTX_O_TERMS bf16 terms for the O projection).
__device__ __forceinline__ void emit_output(float o, int hb, const AttnArgs& a, size_t at) {
  const int lane = threadIdx.x & 63;
  for (int hop = 1; hop < hb; hop <<= 1) {
    const float p = __shfl_xor(o, hop, 64);
    o = (lane & hop) ? p - o : o + p;
  }
  o *= 1.0f / sqrtf((float)hb);
  if (a.out_f32) a.out_f32[at] = o;
  if (a.out_bf16) store_terms<FUTX_O_TERMS>(o, a.out_bf16, at, a.term_stride);
}

// The attention part of the decode block after the QKV projection.  Grid
// (workgroups per sequence, KV heads, sequences); each of the 4 waves of a
// workgroup owns one split of `chunk` tokens:
//   * the wave whose split holds the new token (position L_b) applies RoPE
//     to its key, the block rotation to its key and value, quantizes both
//     per token and writes them to the paged cache at slot L_b; the token's
//     score and value enter the softmax from those same codes in registers
//     (token_blk), so nothing waits on the cache write;
//   * the G query heads of the KV head are rotated (RoPE + block rotation)
//     once per workgroup, head i by wave i % 4, while the first pages' loads
//     are in flight, and reach every wave through LDS as fp16 hi / lo
//     matrix-core fragments;
//   * split-sequence attention over the cached tokens, the four splits of a
//     workgroup merged in LDS into one partial (m, l, acc) per head, which
//     attn_merge_kernel combines across workgroups; when the plan has one
//     workgroup per sequence, the output (inverse rotation included) is
//     written here and no merge runs.
// (Publishing the partials to the last workgroup to arrive, through
// agent-scope coherent stores and an arrival counter, measured slower on
// MI355X than the separate merge launch: 15.1 us against 9.6 + 3.1 us at
// 8B batch 1.)
// Steps from the FuTransformer pages: K/V rotated by a block Hadamard before
// INT4 caching and the rotation undone on the output (kongchang.com/en,
// section "INT4 Decode: letting dequantization feed directly into MMA
// operands"); results written straight into cache locations (same article,
// section "FP8 Prefill: fusing GEMM and epilogue all the way").
// A cached length outside the plan (L_b < 0 or L_b + 1 > tmax) writes
// nothing here (the merge, or this kernel when it finishes, makes that
// group's output NaN).
// (two workgroups per CU: the register budget stays at 256 per lane)
template <int D>
__global__ __launch_bounds__(256, 2) void attn_decode_kernel(AttnArgs a) {
  constexpr int MAXG = 16;  // query heads per KV head (matrix-core columns)
  __shared__ float s_m[4][MAXG], s_l[4][MAXG];
  // rotated queries as fp16 hi / lo (rows padded by 8: the 16 heads' rows
  // start in different LDS banks) and each head's score scale
  __shared__ __align__(16) _Float16 s_qhi[MAXG][D + 8], s_qlo[MAXG][D + 8];
  __shared__ float s_zs[MAXG];
  __shared__ float s_acc[4][MAXG][D];
  const int wg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar
  const int col = lane & 15, grp = lane >> 4;
  const int nkv = a.kv.nkv, G = a.nq / nkv;
  // the table entry of this wave's first page does not depend on the
  // sequence length: its load goes out together with the length's
  const int sp = wg * 4 + wv;
  const int t0 = sp * a.chunk;
  const int32_t* const bt = a.block_table + (size_t)b * a.mpps;
  // the block-table entries of this wave's split, one per lane (lane 63: the
  // sequence's first page, always allocated); clamped into the table row
  const int pg0 = t0 / kPageSize;
  const int btv = bt[lane == 63 ? 0 : min(pg0 + lane, a.mpps - 1)];
  // 1. loads that do not depend on the sequence length go out with it: this
  //    wave's query heads (head wv + 4 k of the group, channel lane + 64 j;
  //    past the group: head 0 again, ignored), the new token's key and value
  //    (every wave loads them, only the owner uses them: unconditional loads
  //    keep the memory-counter waits exact) and the RoPE frequency of the
  //    lane.  Below the length check they would wait for the length's round
  //    trip before their own.
  const float* row = a.qkv + (size_t)b * (a.nq + 2 * nkv) * D;
  constexpr int HPW = MAXG / 4;  // query heads per wave, at most
  float qx[HPW][D / 64];
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int i = wv + 4 * k < G ? wv + 4 * k : 0;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) qx[k][j] = row[(size_t)(h * G + i) * D + lane + 64 * j];
  }
  float kx[D / 64], vx[D / 64];
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    kx[j] = row[(a.nq + h) * D + lane + 64 * j];
    vx[j] = row[(a.nq + nkv + h) * D + lane + 64 * j];
  }
  const double inv_freq = a.inv_freq[lane % (D / 2)];
  const int pos = a.cached_lens[b];  // the new token's position
  const int T = pos + 1;             // tokens attended to
  const size_t obase = ((size_t)b * a.nq + (size_t)h * G) * D;  // output of the group's first head
  if (pos < 0 || T > a.tmax) {
    if (wg == 0 && a.nwg == 1) {
      for (int p = tid; p < G * D; p += 256) {
        if (a.out_f32) a.out_f32[obase + p] = __builtin_nanf("");
        if (a.out_bf16)
#pragma unroll
          for (int t = 0; t < FUTX_O_TERMS; ++t) a.out_bf16[obase + p + t * a.term_stride] = 0x7FC0;
      }
    }
    return;
  }
  const int nsp = (T + a.chunk - 1) / a.chunk;
  const int nwg_b = (nsp + 3) / 4;
  if (wg >= nwg_b) return;  // the whole workgroup, before any barrier
  const KVPtrsConst kvc{a.kv.k_codes, a.kv.v_codes, a.kv.k_scales, a.kv.v_scales, nkv};
  const int t1 = min(t0 + a.chunk, T);
  const bool owner = sp == pos / a.chunk;  // wave-uniform
  const int t1s = owner ? pos : t1;        // cached tokens of the split (the new one comes from registers)

  // 2. the split's first two pages go out first (a wave with nothing to
  //    scan reads the sequence's first page and ignores it: unconditional
  //    loads keep the memory-counter waits exact).  While they are in
  //    flight, each wave rotates its query heads (RoPE + block rotation, the
  //    same steps as for the key) and splits them into fp16 hi / lo at the
  //    head's power-of-two scale; the owner turns the new token into codes.
  //    The fragments reach every wave through LDS.
  const bool scan = t0 < t1s;  // wave-uniform
  KvBlk<D> a0, a1, b0, b1;
  {
    const int pfirst = __builtin_amdgcn_readlane(btv, 63);
    const int p0 = scan ? __builtin_amdgcn_readlane(btv, 0) : pfirst;
    const int p1 = t0 + kPageSize < t1s ? __builtin_amdgcn_readlane(btv, 1) : p0;
    issue_page<D>(kvc, p0, h, a0, a1);
    issue_page<D>(kvc, p1, h, b0, b1);
  }
  float cs, sn;  // cos / sin of frequency index lane % (D / 2), shared by the key and the queries
  rope_cs_inv(pos, inv_freq, &cs, &sn);
  TokenCodes<D> tok;
  if (owner) {
    rope_lane_cs<D>(kx, cs, sn);
    fwht_lane<D>(kx, a.hb);
    fwht_lane<D>(vx, a.hb);
    quantize_token<D>(kx, vx, tok);
  }
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int i = wv + 4 * k;
    if (i < G) {  // wave-uniform
      rope_lane_cs<D>(qx[k], cs, sn);
      fwht_lane<D>(qx[k], a.hb);
      float qmax = 0.f;
#pragma unroll
      for (int j = 0; j < D / 64; ++j) qmax = fmaxf(qmax, fabsf(qx[k][j]));
      qmax = wave_max(qmax);
      const int kq = range_exp(qmax, 11);
#pragma unroll
      for (int j = 0; j < D / 64; ++j) {
        _Float16 hi, lo;
        split_f16(ldexpf(qx[k][j], kq), &hi, &lo);
        s_qhi[i][lane + 64 * j] = hi;
        s_qlo[i][lane + 64 * j] = lo;
      }
      if (lane == 0) s_zs[i] = ldexpf(1.0f, -kq) * (a.scale * kLog2e);
    }
  }
  __syncthreads();
  // matrix-core fragments: lane (grp, col) holds channels 32 s + 8 grp + e
  // of query head col (zero past the group)
  const bool ok = col < G;
  const int qcol = ok ? col : 0;
  f16x8 qh[D / 32], ql[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const f16x8 hv = *(const f16x8*)&s_qhi[qcol][s * 32 + grp * 8];
    const f16x8 lv = *(const f16x8*)&s_qlo[qcol][s * 32 + grp * 8];
    const f16x8 zero = {};
    qh[s] = ok ? hv : zero;
    ql[s] = ok ? lv : zero;
  }
  const float zscale = ok ? s_zs[qcol] : 0.f;

  // 3. this wave's split: the cached tokens, then (owner) the new token
  float m_i = -INFINITY, l_part = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (scan) split_scan<D>(qh, ql, zscale, bt, btv, pg0, t0, t1s, h, kvc, m_i, l_part, acc, a0, a1, b0, b1);
  if (owner) {
    KvBlk<D> nb;
    token_blk<D>(tok, nb);
    compute_blk<D>(pos, T, nb, qh, ql, zscale, m_i, l_part, acc);
    // the cache write goes out last: no later load of this wave waits for it
    const int slot = bt[pos / kPageSize] * kPageSize + pos % kPageSize;
    store_token<D>(tok, slot, h, a.kv);
  }
  float l_tot = l_part + xor_lanes<16>(l_part);
  l_tot += xor_lanes<32>(l_tot);

  // 4. the four splits of the workgroup, merged in LDS
  if (grp == 0 && col < G) {
    s_m[wv][col] = m_i;
    s_l[wv][col] = l_tot;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * grp + r;
    if (i < G) {
#pragma unroll
      for (int cg = 0; cg < D / 64; ++cg)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) s_acc[wv][i][cg * 64 + c4 * 16 + col] = acc[cg * 4 + c4][r];
    }
  }
  __syncthreads();
  // (p = i * D + c: D is a multiple of 64 and the stride 256, so the 64
  //  lanes of a wave always hold 64 consecutive channels of one head)
  auto lds_partial = [&](int i, int c, float& M, float& l, float& acc_c) {
    M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][i]);
    l = 0.f;
    acc_c = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // a wave with no tokens has m = -inf: weight 0
      const float wt = s_m[w][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[w][i] - M);
      l = fmaf(wt, s_l[w][i], l);
      acc_c = fmaf(wt, s_acc[w][i][c], acc_c);
    }
  };
  if (a.nwg == 1) {  // one workgroup per sequence: the output is complete here
    for (int p = tid; p < G * D; p += 256) {
      const int i = p / D, c = p % D;
      float M, l, ac;
      lds_partial(i, c, M, l, ac);
      emit_output(l > 0.f ? ac / l : 0.f, a.hb, a, obase + p);
    }
    return;
  }
  // 5. this workgroup's partial, combined across workgroups by attn_merge_kernel
  const size_t hstride = (size_t)a.nwg * (D + 2);  // between query heads in wpart
  float* const wp = a.wpart + (((size_t)b * a.nq + h * G) * a.nwg + wg) * (D + 2);
  for (int p = tid; p < G * D; p += 256) {
    const int i = p / D, c = p % D;
    float M, l, ac;
    lds_partial(i, c, M, l, ac);
    wp[i * hstride + 2 + c] = ac;
    if (c == 0) {
      wp[i * hstride] = M;
      wp[i * hstride + 1] = l;
    }
  }
}

// Merge of the workgroup partials + inverse block Hadamard.  One block of
// 256 threads per (query head, sequence).  Writes fp32 output, or the
// operand of the O projection: o as an unevaluated sum of FUTX_O_TERMS bf16
// terms (term t at out_bf16 + t * term_stride).  The attention output comes
// out of a long fp32 reduction, so a single bf16 rounding here would flip on
// tiny differences; the terms carry it far below bf16's rounding (gemm.h).
// Thread t owns channel chunk t % (D/4) (four channels) of the partials
// sp = t / (D/4) + (256 / (D/4)) u.  The partials were written by the
// previous kernel on other CUs, so every load of a round (U partials per
// thread) is issued before any is used, and before the sequence length is
// known (indices clamped to the workspace's partials, the extra ones masked
// out afterwards): one round trip per 256 / (D/4) * U partials.  `chunk` is
// the tokens per partial (four attention splits).  A length outside the plan
// (lens[b] < 0 or lens[b] + 1 > tmax) gives a NaN output.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const float* __restrict__ apart, const int32_t* __restrict__ lens, int nq, int chunk, int nsplit,
    int hb, int tmax, float* __restrict__ out_f32, uint16_t* __restrict__ out_bf16, size_t term_stride) {
  constexpr int NC = D / 4;     // float4 chunks per partial
  constexpr int PH = 256 / NC;  // partial phases
  constexpr int U = 4;          // partials per thread and round
  __shared__ float s_m[PH], s_l[PH];
  __shared__ float4 s_acc[PH][NC];
  const int i = blockIdx.x, b = blockIdx.y, t = threadIdx.x, lane = t & 63;
  const int ch = t % NC, ph = t / NC;
  const float* base = apart + ((size_t)b * nq + i) * nsplit * (D + 2);
  // The first round of partials is loaded before the sequence length is
  // known (indices clamped to the plan's splits; partials past the
  // sequence's own splits are never used), so the kernel waits for one
  // memory round trip instead of two.
  float mv[U], lv[U];
  float4 av[U];
  auto load_round = [&](int r0, int lim) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* pw = base + (size_t)min(r0 + ph + PH * u, lim - 1) * (D + 2);
      mv[u] = pw[0];
      lv[u] = pw[1];
      av[u] = *(const float4*)(pw + 2 + 4 * ch);
    }
  };
  load_round(0, nsplit);
  const int L = lens[b] + 1;  // tokens attended to
  if (L < 1 || L > tmax) {
    if (t < D) {
      const size_t at = ((size_t)b * nq + i) * D + t;
      if (out_f32) out_f32[at] = __builtin_nanf("");
      if (out_bf16)
#pragma unroll
        for (int k = 0; k < FUTX_O_TERMS; ++k) out_bf16[at + k * term_stride] = 0x7FC0;
    }
    return;
  }
  float m = -INFINITY, l = 0.f;
  float4 a = {0.f, 0.f, 0.f, 0.f};
  const int nsp = min((L + chunk - 1) / chunk, nsplit);
  for (int r0 = 0; r0 < nsp; r0 += PH * U) {
    if (r0 > 0) load_round(r0, nsp);
    bool ok[U];
    float mr = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ok[u] = r0 + ph + PH * u < nsp;
      if (ok[u]) mr = fmaxf(mr, mv[u]);
    }
    if (mr == -INFINITY) continue;  // no partial of this phase in the round
    const float sc = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mr);
    l *= sc;
    a.x *= sc; a.y *= sc; a.z *= sc; a.w *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = ok[u] ? __builtin_amdgcn_exp2f(mv[u] - mr) : 0.f;
      if (ok[u]) {  // select: a stale partial never enters, not even times 0
        l = fmaf(w, lv[u], l);
        a.x = fmaf(w, av[u].x, a.x);
        a.y = fmaf(w, av[u].y, a.y);
        a.z = fmaf(w, av[u].z, a.z);
        a.w = fmaf(w, av[u].w, a.w);
      }
    }
    m = mr;
  }
  if (ch == 0) {
    s_m[ph] = m;
    s_l[ph] = l;
  }
  s_acc[ph][ch] = a;
  __syncthreads();
  if (t >= D) return;
  // channel c = t: the phases merged in a fixed order (phase 0 always holds
  // partial 0, so M is finite)
  const int c = t;
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < PH; ++p) M = fmaxf(M, s_m[p]);
  float o = 0.f, ltot = 0.f;
#pragma unroll
  for (int p = 0; p < PH; ++p) {
    const float w = s_m[p] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[p] - M);
    o = fmaf(w, ((const float*)&s_acc[p][c / 4])[c % 4], o);
    ltot = fmaf(w, s_l[p], ltot);
  }
  o = ltot > 0.f ? o / ltot : 0.f;
  // inverse rotation (the normalized Sylvester matrix is its own inverse)
  for (int hop = 1; hop < hb; hop <<= 1) {
    const float p = __shfl_xor(o, hop, 64);
    o = (lane & hop) ? p - o : o + p;
  }
  o *= 1.0f / sqrtf((float)hb);
  if (out_f32) out_f32[((size_t)b * nq + i) * D + c] = o;
  if (out_bf16)  // o as FUTX_O_TERMS bf16 terms, the O projection operand
    store_terms<FUTX_O_TERMS>(o, out_bf16, (size_t)b * nq * D + (size_t)i * D + c, term_stride);
}

// ---------------------------------------------------------------- launchers

#define FUTX_LAUNCH_CHECK()                                   \
  do {                                                        \
    hipError_t e_ = hipGetLastError();                        \
    if (e_ != hipSuccess) return e_;                          \
  } while (0)

hipError_t launch_prep_act(const float* x, int B, int H, float eps, uint16_t* act, float* invr,
                           hipStream_t st) {
  if (H % 128) return hipErrorInvalidValue;
  prep_act_kernel<<<B, 1024, 0, st>>>(x, H, eps, act, invr);
  FUTX_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_reduce(const float* part, int S, int B, int N, const float* rowscale,
                         const float* resid, float* out, int gateup_inter, hipStream_t st) {
  const int total = B * N;
  reduce_kernel<<<(total + 255) / 256, 256, 0, st>>>(part, S, B, N, rowscale, resid, out, gateup_inter);
  FUTX_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_swiglu(const float* part, int S, int B, int I, const float* invr, uint16_t* act,
                         hipStream_t st) {
  swiglu_kernel<<<dim3((I + 255) / 256, B), 256, 0, st>>>(part, S, B, I, invr, act);
  FUTX_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_kv_append(const float* k, const float* v, const int32_t* positions,
                            const int32_t* slots, int n, uint32_t flags, int D, int hb,
                            float theta, const KVPtrs& kv, hipStream_t st) {
  const dim3 grid(n, kv.nkv);
  if (D == 128)
    kv_append_kernel<128><<<grid, 64, 0, st>>>(k, v, positions, slots, flags, hb, theta, kv);
  else
    kv_append_kernel<64><<<grid, 64, 0, st>>>(k, v, positions, slots, flags, hb, theta, kv);
  FUTX_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_attn_decode(AttnArgs a, int B, int D, const AttnPlan& plan, hipStream_t st) {
  if (a.nq % a.kv.nkv != 0 || a.nq / a.kv.nkv > 16) return hipErrorInvalidValue;
  a.chunk = plan.chunk;
  a.nwg = (plan.nsplit + 3) / 4;
  a.scale = 1.0f / sqrtf((float)D);
  // RoPE inverse frequencies theta^(-2i/D) in fp64, the same expression as
  // the RoPE definition evaluates (the kernels take the angle pos * inv)
  for (int i = 0; i < 64; ++i) a.inv_freq[i] = i < D / 2 ? std::pow((double)a.theta, -2.0 * i / (double)D) : 0.0;
  const dim3 grid(a.nwg, a.kv.nkv, B);
  if (D == 128)
    attn_decode_kernel<128><<<grid, 256, 0, st>>>(a);
  else
    attn_decode_kernel<64><<<grid, 256, 0, st>>>(a);
  FUTX_LAUNCH_CHECK();
  if (a.nwg == 1) return hipSuccess;  // finished in the attention kernel
  // the workgroup partials: 4 * chunk tokens each
  const dim3 mgrid(a.nq, B);
  if (D == 128)
    attn_merge_kernel<128><<<mgrid, 256, 0, st>>>(a.wpart, a.cached_lens, a.nq, 4 * a.chunk, a.nwg, a.hb,
                                                   a.tmax, a.out_f32, a.out_bf16, a.term_stride);
  else
    attn_merge_kernel<64><<<mgrid, 256, 0, st>>>(a.wpart, a.cached_lens, a.nq, 4 * a.chunk, a.nwg, a.hb, a.tmax,
                                                  a.out_f32, a.out_bf16, a.term_stride);
  FUTX_LAUNCH_CHECK();
  return hipSuccess;
}

#ifndef FUTX_ATTN_SPLITS
#define FUTX_ATTN_SPLITS 2048
#endif

AttnPlan attn_plan(int B, int nkv, int max_context) {
  AttnPlan p;
  const int pages = (max_context + kPageSize - 1) / kPageSize;
  const long work = (long)B * nkv * pages;  // page-sized work items
  // pages per split: at most FUTX_ATTN_SPLITS splits (waves) in total
  int cp = (int)((work + FUTX_ATTN_SPLITS - 1) / FUTX_ATTN_SPLITS);
  cp = cp < 1 ? 1 : cp;
  p.chunk = cp * kPageSize;
  p.nsplit = (max_context + p.chunk - 1) / p.chunk;
  if (p.nsplit < 1) p.nsplit = 1;
  return p;
}

// attn_plan(B, nkv, c).nsplit <= this bound for every c <= max_context: with
// one page per split nsplit = pages <= FUTX_ATTN_SPLITS / (B nkv); with more,
// pages / chunk pages <= FUTX_ATTN_SPLITS / (B nkv).  The bound does not
// decrease with the context, so a workspace sized with it fits every shorter
// context too.
int attn_nsplit_bound(int B, int nkv, int max_context) {
  const long pages = (max_context + kPageSize - 1) / kPageSize;
  const long cap = (FUTX_ATTN_SPLITS + (long)B * nkv - 1) / ((long)B * nkv);
  const long n = pages < cap ? pages : cap;
  return n < 1 ? 1 : (int)n;
}

}  // namespace futx
