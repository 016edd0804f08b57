// Host weight packer: gain folding, fp32 round-to-nearest INT4 quantization
// and the reorder into matrix-core operand order (layout.h).
//
// The pages fix INT4 projection weights quantized by round-to-nearest and
// the folding of the fixed RMSNorm gain into the weights that follow the
// norm (FuTransformer abstract, airebao.com item page; article
// kongchang.com/en, sections "FP8 Prefill: fusing GEMM and epilogue all the
// way" and "Accuracy cost: perplexity from 6.24 to 7.23").  Group size,
// scale type and rounding are readings: one fp16 scale max|w|/7 per group of
// w_group inputs, computed in fp32, ties to even, the stored scale as the
// divisor, codes clamped to [-8, 7].
#include <atomic>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "internal.h"

namespace futx {
namespace {

// IEEE binary16 of an fp32 value, round to nearest even.
uint16_t f32_to_f16_rne(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return (uint16_t)(sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u));
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);  // >= 65520 rounds to inf
  int e = (int)(ax >> 23);
  uint32_t m = (ax & 0x7FFFFFu) | 0x800000u;
  if (e < 113) {  // below 2^-14: binary16 subnormal, unit 2^-24
    if (e < 102) return (uint16_t)sign;  // < 2^-25 rounds to zero
    int shift = 126 - e;                 // value / 2^-24 = m * 2^(e - 126)
    uint32_t q = m >> shift, rem = m & ((1u << shift) - 1), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    return (uint16_t)(sign | q);
  }
  uint32_t e16 = (uint32_t)(e - 112);
  uint32_t m10 = (ax & 0x7FFFFFu) >> 13, rem = ax & 0x1FFFu;
  uint32_t h = (e16 << 10) + m10;
  if (rem > 0x1000u || (rem == 0x1000u && (m10 & 1))) ++h;  // carry may bump the exponent
  return (uint16_t)(sign | h);
}

float f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
  float v;
  if (e == 0) {
    v = std::ldexp((float)m, -24);
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = std::ldexp((float)(m | 0x400), (int)e - 25);
  }
  uint32_t bits;
  std::memcpy(&bits, &v, 4);
  bits |= sign;
  std::memcpy(&v, &bits, 4);
  return v;
}

struct PackJob {
  const futx_dims* d;
  futx_proj proj;
  const float* w;
  const float* gain;
  uint8_t* packed;
  uint16_t* scales;
  int n, k, group, kblocks;
};

// Quantizes logical rows [r0, r1); returns false on fp16 overflow.
bool pack_rows(const PackJob& j, int r0, int r1) {
  std::vector<float> row(j.k);
  std::vector<int8_t> q(j.k);
  const int ngroups = j.k / j.group;
  for (int n = r0; n < r1; ++n) {
    const float* src = j.w + (size_t)n * j.k;
    for (int c = 0; c < j.k; ++c) row[c] = j.gain ? src[c] * j.gain[c] : src[c];
    const int P = j.proj == FUTX_PROJ_GATEUP ? gateup_physical_row(n, j.d->intermediate) : n;
    for (int g = 0; g < ngroups; ++g) {
      const float* x = row.data() + (size_t)g * j.group;
      float a = 0.f;
      for (int c = 0; c < j.group; ++c) a = std::fmax(a, std::fabs(x[c]));
      uint16_t s16 = f32_to_f16_rne(a / 7.0f);
      if ((s16 & 0x7C00u) == 0x7C00u) return false;
      j.scales[scale_index(P, g, j.kblocks, j.group)] = s16;
      float sf = f16_to_f32(s16);
      for (int c = 0; c < j.group; ++c) {
        float v = sf == 0.f ? 0.f : std::nearbyint(x[c] / sf);
        v = std::fmin(std::fmax(v, -8.f), 7.f);
        q[(size_t)g * j.group + c] = (int8_t)v;
      }
    }
    for (int c = 0; c < j.k; ++c) {
      size_t off;
      int e;
      weight_nibble_pos(P, c, j.kblocks, &off, &e);
      uint32_t word;
      std::memcpy(&word, j.packed + off, 4);
      word = nibble_put(word, e, (uint32_t)(q[c] + (int)kNibbleBias));
      std::memcpy(j.packed + off, &word, 4);
    }
  }
  return true;
}

}  // namespace

futx_status pack_host(const futx_dims* dims, futx_proj proj, const float* w, const float* gain,
                      void* packed, void* scales) {
  futx_status st = check_dims(dims);
  if (st) return st;
  if ((st = check_proj(proj))) return st;
  if (!w || !packed || !scales) return fail(FUTX_E_ARG, "pack: null pointer");
  ProjShape ps = proj_shape(*dims, proj);
  PackJob j{dims, proj, w, gain, (uint8_t*)packed, (uint16_t*)scales, ps.n, ps.k, dims->w_group,
            ps.k / kTileK};
  std::memset(scales, 0, 2 * scale_count(ps.n, ps.k / kTileK, dims->w_group));  // padding
  // Rows of one 16-row tile share 32-bit words, so threads own whole tiles
  // (GATEUP: a logical tile maps to one physical tile).
  const int tiles = ps.n / kTileN;
  unsigned hw = std::thread::hardware_concurrency();
  int nthreads = (int)std::min<unsigned>(hw ? hw : 1, 32);
  if ((size_t)ps.n * ps.k < (1u << 20)) nthreads = 1;
  std::atomic<bool> ok{true};
  std::atomic<int> next{0};
  auto worker = [&]() {
    for (;;) {
      int t = next.fetch_add(1);
      if (t >= tiles || !ok.load()) return;
      if (!pack_rows(j, t * kTileN, (t + 1) * kTileN)) ok = false;
    }
  };
  std::vector<std::thread> pool;
  for (int i = 1; i < nthreads; ++i) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
  if (!ok) return fail(FUTX_E_RANGE, "pack: a group scale max|w|/7 overflows fp16");
  return FUTX_OK;
}

futx_status pack_codes_host(const futx_dims* dims, futx_proj proj, const uint8_t* canon,
                            const uint16_t* canon_scales, void* packed, void* scales) {
  futx_status st = check_dims(dims);
  if (st) return st;
  if ((st = check_proj(proj))) return st;
  if (!canon || !canon_scales || !packed || !scales) return fail(FUTX_E_ARG, "pack_codes: null pointer");
  ProjShape ps = proj_shape(*dims, proj);
  const int kblocks = ps.k / kTileK, ngroups = ps.k / dims->w_group;
  for (size_t i = 0; i < (size_t)ps.n * ngroups; ++i)
    if ((canon_scales[i] & 0x7C00u) == 0x7C00u)
      return fail(FUTX_E_RANGE, "pack_codes: scale %zu is not a finite fp16 value", i);
  uint8_t* pk = (uint8_t*)packed;
  uint16_t* sc = (uint16_t*)scales;
  std::memset(scales, 0, 2 * scale_count(ps.n, kblocks, dims->w_group));  // padding
  for (int n = 0; n < ps.n; ++n) {
    const int P = proj == FUTX_PROJ_GATEUP ? gateup_physical_row(n, dims->intermediate) : n;
    for (int g = 0; g < ngroups; ++g)
      sc[scale_index(P, g, kblocks, dims->w_group)] = canon_scales[(size_t)n * ngroups + g];
    for (int c = 0; c < ps.k; ++c) {
      // canonical byte: element 2i in the low nibble, 2i + 1 in the high
      // nibble, two's-complement codes in [-8, 7]
      const uint32_t nib = (canon[(size_t)n * (ps.k / 2) + c / 2] >> (4 * (c & 1))) & 15u;
      const int code = (int)(nib ^ 8u) - 8;
      size_t off;
      int e;
      weight_nibble_pos(P, c, kblocks, &off, &e);
      uint32_t word;
      std::memcpy(&word, pk + off, 4);
      word = nibble_put(word, e, (uint32_t)(code + (int)kNibbleBias));
      std::memcpy(pk + off, &word, 4);
    }
  }
  return FUTX_OK;
}

futx_status unpack_host(const futx_dims* dims, futx_proj proj, const void* packed,
                        const void* scales, uint8_t* canon, uint16_t* canon_scales) {
  ProjShape ps = proj_shape(*dims, proj);
  const int kblocks = ps.k / kTileK, ngroups = ps.k / dims->w_group;
  const uint8_t* pk = (const uint8_t*)packed;
  const uint16_t* sc = (const uint16_t*)scales;
  for (int n = 0; n < ps.n; ++n) {
    const int P = proj == FUTX_PROJ_GATEUP ? gateup_physical_row(n, dims->intermediate) : n;
    for (int g = 0; g < ngroups; ++g)
      canon_scales[(size_t)n * ngroups + g] = sc[scale_index(P, g, kblocks, dims->w_group)];
    for (int c = 0; c < ps.k; c += 2) {
      uint8_t nib[2];
      for (int t = 0; t < 2; ++t) {
        size_t off;
        int e;
        weight_nibble_pos(P, c + t, kblocks, &off, &e);
        uint32_t word;
        std::memcpy(&word, pk + off, 4);
        int code = (int)nibble_get(word, e) - (int)kNibbleBias;
        nib[t] = (uint8_t)(code & 0xF);
      }
      canon[(size_t)n * (ps.k / 2) + c / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
    }
  }
  return FUTX_OK;
}

futx_status fold_head_host(int32_t vocab, int32_t hidden, const uint16_t* w, const float* gain,
                           uint16_t* out) {
  if (vocab <= 0 || hidden <= 0 || !w || !gain || !out) return fail(FUTX_E_ARG, "fold_head: bad args");
  for (size_t r = 0; r < (size_t)vocab; ++r) {
    for (int c = 0; c < hidden; ++c) {
      uint32_t bits = (uint32_t)w[r * hidden + c] << 16;
      float f;
      std::memcpy(&f, &bits, 4);
      f = f * gain[c];
      std::memcpy(&bits, &f, 4);
      // bf16 round to nearest even (finite inputs)
      uint32_t lsb = (bits >> 16) & 1u;
      bits += 0x7FFFu + lsb;
      out[r * hidden + c] = (uint16_t)(bits >> 16);
    }
  }
  return FUTX_OK;
}

}  // namespace futx
