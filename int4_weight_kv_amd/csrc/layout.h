// Memory layouts shared by the host packer and the gfx950 kernels.
//
// Matrix-core operand order.  The kernels multiply with
// v_mfma_f32_16x16x32_bf16: lane L of a wave holds, for one 16 x 32 operand,
// row (L % 16) and the 8 consecutive reduction indices 8 * (L / 16) .. +7;
// the 16 x 16 fp32 result gives lane L rows 4 * (L / 16) + r (r = 0..3) of
// column L % 16.  Weights and keys are stored so that one 128-bit load per
// lane yields exactly its operand nibbles for four consecutive MFMA steps,
// which are then widened to bf16 in registers (no tile is written back),
// following the pages' design of feeding dequantized values straight into
// the matrix cores (FuTransformer abstract, airebao.com item page; article
// kongchang.com/en, section "INT4 Decode: letting dequantization feed
// directly into MMA operands").
//
// Nibble encoding inside a 32-bit word: a word carries operand elements
// e = 0..7 of one lane and one MFMA step.  Element e is stored as
// n = code + 8 in bits 3..6 rotated left by r(e) = 4 (e / 2) + 16 (e % 2)
// (so element 7 wraps around bit 31).  For the element pair j = (2j, 2j+1),
//   (rotr(w, 4j) & 0x00780078) | 0x41804180
// is a pair of bf16 values 16 + n = 24 + code (exponent 2^4, the nibble in
// mantissa bits 3..6): two elements per two ALU instructions (one for
// j = 0), no conversion instruction.  The constant 24 is removed after the
// MFMA with the sums of the other operand:
//   sum_k (24 + q_k) a_k = sum_k q_k a_k + 24 sum_k a_k.
// The offset is kept small (24 rather than 136 for a nibble in the low
// mantissa bits) because the fp32 rounding of the MFMA sum scales with it.
// Weights (one projection, N physical rows x K inputs, group G along K):
//   packed[nt][kb][L][16 bytes], nt = row tile (16 rows), kb = K block (128),
//   word s (bytes 4s..4s+3) of lane L holds row nt*16 + L%16 and inputs
//   kb*128 + 32 s + 8 (L/16) + e.
//   scales fp16 [nt][kb / 8][i 16][8 * 128 / G]: row P = nt*16 + i, group g
//   of K block kb = g * G / 128 at position (kb % 8) * 128 / G + g % (128 / G).
// Physical rows equal logical rows except GATEUP, whose 16-row tiles
// alternate gate / up: physical tile 2t holds gate rows 16t..16t+15 and
// tile 2t+1 holds up rows 16t..16t+15, so one wave sees both halves of a
// SwiGLU column block.
//
// KV cache (per layer, page of 64 tokens, per KV head):
//   k_codes[page][h][tt][L][D/8 bytes]  tt = token tile (16 tokens);
//     lane L holds token tt*16 + L%16, word s holds channels
//     32 s + 8 (L/16) + e  (the key is the 16-row A operand of q.k).
//   v_codes[page][h][tb][cg][L][16 bytes]  tb = token block (32 tokens),
//     cg = channel group (64 channels); word c4 holds channel
//     cg*64 + 16 c4 + L%16 and tokens tb*32 + tok(L/16, e) with
//     tok(g, e) = 4g + e (e < 4) or 16 + 4g + (e - 4) (e >= 4): this is the
//     order in which the q.k result tiles of tokens 0-15 and 16-31 come out
//     of the MFMA, so scores feed p.v without a transpose.
//   k_scales / v_scales[page][h][64] fp16.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace futx {

constexpr int kTileN = 16;       // weight rows per tile
constexpr int kTileK = 128;      // inputs per K block
constexpr int kTileBytes = 1024; // 16 x 128 nibbles
constexpr int kPageSize = 64;
constexpr int kMaxBatch = 32;
constexpr uint32_t kNibbleBias = 8;

inline size_t weight_tile_offset(int nt, int kb, int kblocks) {
  return ((size_t)nt * kblocks + kb) * kTileBytes;
}

inline uint32_t rotl32(uint32_t x, int r) {
  r &= 31;
  return r ? (x << r) | (x >> (32 - r)) : x;
}
inline int nibble_rot(int e) { return 4 * (e >> 1) + 16 * (e & 1); }
// word with element e set to nibble n (0..15)
inline uint32_t nibble_put(uint32_t w, int e, uint32_t n) {
  const int r = nibble_rot(e);
  return (w & ~rotl32(0x78u, r)) | rotl32((n & 15u) << 3, r);
}
inline uint32_t nibble_get(uint32_t w, int e) { return (rotl32(w, 32 - nibble_rot(e)) >> 3) & 15u; }

// byte offset of the word and element index of (physical row P, input k)
inline void weight_nibble_pos(int P, int k, int kblocks, size_t* word_off, int* elem) {
  int nt = P / kTileN, i = P % kTileN;
  int kb = k / kTileK, kk = k % kTileK;
  int s = kk / 32, g = (kk % 32) / 8, e = kk % 8;
  int lane = g * 16 + i;
  *word_off = weight_tile_offset(nt, kb, kblocks) + (size_t)lane * 16 + (size_t)s * 4;
  *elem = e;
}

// Group scales, fp16, blocked by weight tile: [nt][kb / 8][row i 16][groups
// of those 8 K blocks], i.e. 8 * 128 / group scales per (tile row, 8 K
// blocks), the last block padded when the K block count is not a multiple
// of 8.  One tile's 16 scales share a 32-byte (group 128) run.
inline int scale_kb_blocks(int kblocks) { return (kblocks + 7) / 8; }
inline size_t scale_count(int n, int kblocks, int group) {
  return (size_t)n * scale_kb_blocks(kblocks) * 8 * (kTileK / group);
}
inline size_t scale_index(int P, int g, int kblocks, int group) {
  const int per_kb = kTileK / group, seg = 8 * per_kb;
  const int nt = P / kTileN, i = P % kTileN, kb = g / per_kb, gi = g % per_kb;
  return (((size_t)nt * scale_kb_blocks(kblocks) + kb / 8) * kTileN + i) * seg + (kb % 8) * per_kb + gi;
}

// GATEUP: physical row of logical row n (0..2I-1); identity for the others.
inline int gateup_physical_row(int n, int inter) {
  int half = n / inter, r = n % inter;
  return (2 * (r / kTileN) + half) * kTileN + r % kTileN;
}
inline int gateup_logical_row(int P, int inter) {
  int p = P / kTileN, i = P % kTileN;
  return (p % 2) * inter + (p / 2) * kTileN + i;
}

}  // namespace futx
