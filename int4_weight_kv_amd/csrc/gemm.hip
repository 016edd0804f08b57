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
// tiles; for the SwiGLU projection gate/up tile pairs) over one K range, and
// each of its NW waves (4, or 8 for long K with few items) owns 1 / NW of
// that K range (its "quarter" below) for every item.  A
// wave first stages its own quarter of the activation (all batch rows) in
// LDS as bf16 matrix-core operands (an fp32 source is rounded to bf16 there,
// which is the RMSNorm operand rounding), together with the exact (fp64) sum
// of those operands per weight group, which removes the nibble offset, and
// for an fp32 source the partial RMSNorm sum of squares; no barrier is
// needed, since a wave reads only what it wrote.  The activation loads go
// out before the weight loads and are converted while the weights stream.
// Then the wave streams its quarter of item after item: 128-bit loads, 16
// bytes per lane per 1 KB tile, in chunks of eight tiles (four for gate/up
// pairs or batches above 16) with the next chunk in flight across item
// boundaries.  At the end of an item the NW wave sums are added in LDS
// and one wave (rotating) keeps them; the epilogue and the only global
// stores run after the last item.
//
// Every vector load of the main loop is unconditional: loads complete in
// order, so the compiler's wait before a use then covers exactly the loads
// issued before it, and the chunk after the one in use stays in flight.
#include <algorithm>
#include <type_traits>

#include "device.h"
#include "gemm.h"

#ifndef FUTX_GEMM_WIDE_NW
#define FUTX_GEMM_WIDE_NW 16  // waves per workgroup when items are few (4, 8 or 16)
#endif
#ifndef FUTX_GEMM_OCC
#define FUTX_GEMM_OCC 3  // workgroups per CU the item split aims at (batch <= 4)
#endif
#ifndef FUTX_GEMM_OCC_BATCH
#define FUTX_GEMM_OCC_BATCH 1  // the same for batches above 4
#endif
#ifndef FUTX_GEMM_DEEP_MIN_B
#define FUTX_GEMM_DEEP_MIN_B 5  // smallest batch whose fused epilogues need 16-wave workgroups
#endif
#ifndef FUTX_GEMM_WIDE_PCT
#define FUTX_GEMM_WIDE_PCT 100  // "few": items <= this percentage of the CU count
#endif

namespace futx {

// floor(x / d) for 0 <= x < 2^20 and d >= 1, from a reciprocal taken once
// per divisor: the fp32 estimate x * rcp(d) is within 1/4 of x / d (the
// reciprocal is within 1 ulp, x is exact in fp32), so its truncation is off
// by at most one, which the two corrections remove.  Six instructions
// instead of the thirty or so of the compiler's general 32-bit division,
// which the kernel needs for every chunk and many staging addresses.
struct SmallDiv {
  int d;
  float r;
  __device__ explicit SmallDiv(int d_) : d(d_), r(__builtin_amdgcn_rcpf((float)d_)) {}
  __device__ int div(int x) const {
    int q = (int)((float)x * r);
    q -= q * d > x ? 1 : 0;
    q += (q + 1) * d <= x ? 1 : 0;
    return q;
  }
};

// Register budget: at most three waves per SIMD for 4- and 8-wave
// workgroups (more would make the compiler spill the prologue's staging
// registers); a 16-wave workgroup (one per CU, four waves per SIMD) streams
// chunks of two K blocks, which keeps it within 128 registers.
template <int G, int NF, int NR, int NT, bool F32, int EPI, int PAIR, int NW>
__global__ __launch_bounds__(64 * NW, (NW < 16 && NF == 1 && G == 128) ? 2 : 1)
__attribute__((amdgpu_waves_per_eu(NW == 16 ? 4 : 1, NW == 16 ? 4 : 3))) void int4_gemm_kernel(GemmArgs a) {
  constexpr int NTH = 64 * NW;                       // threads per workgroup
  constexpr int NTW = PAIR ? 2 : 1;                  // weight tiles per item (gate + up)
  constexpr int CHK = NW == 16 ? 2 : (PAIR || NF == 2) ? 4 : 8;  // K blocks per chunk and wave
  // activation passes held in registers (one L2 round trip each batch of
  // MAXP); fp32 rows of more than 4 sequences take 8 as well, except in
  // 16-wave workgroups (register budget; two round trips of 4 measured no
  // slower there)
  constexpr int MAXP = NW == 16 ? 4 : ((!F32 && NT == 1) || (F32 && NR >= 2)) ? 8 : 4;
  extern __shared__ __align__(16) uint8_t s_dyn[];
  // LDS (gemm_lds_layout): activation range [NT][B][row] bf16 | group sums
  // [B][ngr] float2 | group sums of squares [B][ngr] | partials
  // [2][4][NTW][NF][NR][64] | ss [B] | item sums [item - it0][NTW][B][16] |
  // scales
  const int tid = threadIdx.x, lane = tid & 63;
  const int wq = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (0..NW-1), scalar
  const int col = lane & 15, grp = lane >> 4;
  // Batch tiles: workgroup w of tile t runs as block ((w / 8) * ntiles + t)
  // * 8 + w % 8.  Blocks go to the 8 XCDs in turn, so the tiles of one item
  // run sit on one XCD at the same time and read the weights through its L2
  // (one HBM read).  Blocks past the plan (grid padding) leave at once.
  int wgi = blockIdx.x, b0 = 0, B = a.B;  // B: rows of the tile, b0: its first row
  const int ntl = a.ntiles > 1 ? a.ntiles : 1;
  if (ntl > 1) {
    const SmallDiv dt(ntl);
    const int r = wgi >> 3, rq = __builtin_amdgcn_readfirstlane(dt.div(r)), bt = r - rq * ntl;
    wgi = rq * 8 + (wgi & 7);
    b0 = __builtin_amdgcn_readfirstlane(dt.div(bt * a.B));
    B = __builtin_amdgcn_readfirstlane(dt.div((bt + 1) * a.B)) - b0;
  }
  if (wgi >= a.splits * a.wgs_per_split) return;
  const int KB = a.K >> 7;
  const int split = __builtin_amdgcn_readfirstlane(SmallDiv(a.wgs_per_split).div(wgi));
  const int wj = wgi - split * a.wgs_per_split;
  const int kb0 = split * a.kb_per_wg, kb1 = min(kb0 + a.kb_per_wg, KB);
  const int krange = kb1 - kb0;
  const int it0 = (int)((unsigned)wj * (unsigned)a.items / (unsigned)a.wgs_per_split);
  const int it1 = (int)((unsigned)(wj + 1) * (unsigned)a.items / (unsigned)a.wgs_per_split);
  const int row = krange * 128 + 8;  // bf16 elements per LDS row (16 B pad)
  const int ngr = krange * 128 / G;
  constexpr int SEG = 8 * (128 / G);  // scales per (row, 8 K blocks)
  const int KB8 = (KB + 7) >> 3;
  const int b80 = kb0 >> 3, nkb8 = ((kb1 + 7) >> 3) - b80;
  const GemmLds L = gemm_lds_layout(NT, B, krange, G, NTW, NF * NR, it1 - it0, nkb8, NW);
  uint16_t* const s_act = (uint16_t*)(s_dyn + L.act);
  float2* const s_gsum = (float2*)(s_dyn + L.gsum);
  float* const s_sqg = (float*)(s_dyn + L.sqg);
  float* const s_part = (float*)(s_dyn + L.part);
  float* const s_ss = (float*)(s_dyn + L.ss);
  float* const s_out = (float*)(s_dyn + L.out);
  // scales of the workgroup's items over its K range, blocked as in global
  // memory: [item - it0][NTW][kb / 8 - kb0 / 8][row 16][SEG]
  uint16_t* const s_scl = (uint16_t*)(s_dyn + L.scl);

  // this wave's share (1 / NW) of the K range, in chunks of CHK K blocks
  const int kbq = (krange + NW - 1) / NW;
  const int q0 = min(kb0 + wq * kbq, kb1), q1 = min(q0 + kbq, kb1);
  const int cpi = (kbq + CHK - 1) / CHK;  // chunks per item (same for every wave)
  const SmallDiv dcpi(cpi > 0 ? cpi : 1), dbr(B * 16);
  // item offset of chunk c (uniform)
  auto citem = [&](int c) { return __builtin_amdgcn_readfirstlane(dcpi.div(c)); };
  const int nchunks = (it1 - it0) * cpi;
  if (nchunks == 0) return;  // the whole workgroup: before any barrier

  // Residual of the first write-out pass, loaded before anything else so the
  // epilogue does not start a dependent round trip (oldest load: waiting for
  // it never waits for a weight load).  Clamped, unconditional.
  float resid_pf = 0.f;
  if constexpr (EPI == kEpiResid) {
    const int idx = min(tid, (it1 - it0) * B * 16 - 1);
    const int il = dbr.div(idx), rem = idx - il * B * 16;
    resid_pf = a.resid[(size_t)(b0 + (rem >> 4)) * a.N + (it0 + il) * 16 + (rem & 15)];
  }

  // ---- weights: the main loop issues weight loads only (scales come from LDS)
  uint4 wA[CHK][NTW], wB[CHK][NTW];
  // Out-of-range K blocks of a chunk re-read the quarter's first block and
  // are weighted by zero.
  auto load_chunk = [&](uint4 (&w)[CHK][NTW], int c) {
    const int ci = citem(c);
    const int item = it0 + ci, cb = q0 + (c - ci * cpi) * CHK;
#pragma unroll
    for (int i = 0; i < CHK; ++i) {
      const int kb = cb + i < q1 ? cb + i : (q0 < q1 ? q0 : kb0);
#pragma unroll
      for (int u = 0; u < NTW; ++u) {
        const int nt = PAIR ? 2 * item + u : item;
        const uint4* wt = a.w + ((size_t)nt * KB + kb) * 64;
        w[i][u] = wt[lane];
      }
    }
  };

  // ---- scale staging: 16-byte pieces; piece p = ((il * NTW + u) * nkb8 +
  // j) * 16 * (SEG / 8) + r covers row r / (SEG / 8), part r % (SEG / 8)
  constexpr int MAXS = 4;  // pieces per thread held in registers
  const int npieces = (it1 - it0) * NTW * nkb8 * 16 * (SEG / 8);
  const SmallDiv dnkb(nkb8 > 0 ? nkb8 : 1);
  auto scl_src = [&](int p) -> const uint4* {
    const int per_blk = 16 * (SEG / 8);
    const int blk = p / per_blk, r = p - blk * per_blk;
    const int iu = dnkb.div(blk), j = blk - iu * nkb8;
    const int nt = PAIR ? 2 * (it0 + iu / NTW) + iu % NTW : it0 + iu;
    return (const uint4*)(a.sc + ((size_t)nt * KB8 + b80 + j) * 16 * SEG) + r;
  };

  // ---- activation staging of this wave's quarter: the quarter's rows
  // [B][qk] are taken as one run of B * qk elements, pass p covering
  // [p * 512, +512), 8 per lane.  qk is a multiple of 128, so the G / 8
  // lanes of a weight group always sit in one row.
  const int qk = (q1 - q0) * 128;
  const int nelem = B * qk;
  const SmallDiv dqk(qk > 0 ? qk >> 7 : 1);
  const int npass = (nelem + 511) >> 9;
  // (row, element) of this lane in pass p; lanes past the end read row 0
  auto act_pos = [&](int p, int& b, int& e) {
    const int f = p * 512 + lane * 8;
    const int fc = f < nelem ? f : 0;
    b = qk ? dqk.div(fc >> 7) : 0;  // qk is a multiple of 128
    e = fc - b * qk;
  };
  using ActRegs = typename std::conditional<F32, float4[2], uint4[NT]>::type;
  auto act_load = [&](int p, ActRegs& r) {  // p < 0 (empty quarter): row 0, a valid address
    int b, e;
    act_pos(p < 0 ? 0 : p, b, e);
    const size_t src = (size_t)(b0 + b) * a.K + q0 * 128 + e;
    if constexpr (F32) {
      const float4* q = (const float4*)((const float*)a.act + src);
      r[0] = q[0];
      r[1] = q[1];
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) r[t] = *(const uint4*)((const uint16_t*)a.act + t * a.term_stride + src);
    }
  };
  // valid == false (wave-uniform): the pass is past the end (registers hold
  // a repeated pass) and is skipped.  Callers derive the flag so that the
  // compiler cannot turn the guarded unrolled loop into an early-exit loop
  // over a dynamically indexed register array (scratch).
  auto act_store = [&](int p, const ActRegs& r, bool valid) {
    if (!valid) return;
    int b, e;
    act_pos(p, b, e);
    const bool ok = p * 512 + lane * 8 < nelem;
    const int kl = (q0 - kb0) * 128 + e;  // offset in the workgroup's K range
    double gs = 0.0;
    float sq = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint4 v;
      if constexpr (F32) {
        const float4 x0 = r[0], x1 = r[1];
        v = uint4{pack2_bf16(x0.x, x0.y), pack2_bf16(x0.z, x0.w), pack2_bf16(x1.x, x1.y), pack2_bf16(x1.z, x1.w)};
        sq = fmaf(x0.x, x0.x, fmaf(x0.y, x0.y, fmaf(x0.z, x0.z, fmaf(x0.w, x0.w, sq))));
        sq = fmaf(x1.x, x1.x, fmaf(x1.y, x1.y, fmaf(x1.z, x1.z, fmaf(x1.w, x1.w, sq))));
      } else {
        v = r[t];
      }
      if (ok) *(uint4*)(s_act + (size_t)(t * B + b) * row + kl) = v;
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        gs += (double)bf16_bits_to_f32(w4[c] & 0xFFFF) + (double)bf16_bits_to_f32(w4[c] >> 16);
    }
    // a weight group is G / 8 consecutive lanes
    gs = group_sum<G / 8>(gs);
    if constexpr (F32) sq = group_sum<G / 8>(sq);
    if (ok && (lane % (G / 8)) == 0) {
      s_gsum[(size_t)b * ngr + kl / G] = split_f64(gs);
      if constexpr (F32) s_sqg[(size_t)b * ngr + kl / G] = sq;
    }
  };

  // Batch placement in the matrix-core tile: A row `col` of fragment f holds
  // batch 16f + 4(col % 4) + col / 4, so D register r of lane group grp holds
  // batch 16f + 4r + grp and a batch of at most 4 needs D register 0 only.
  // A rows past the batch repeat a valid row; their results are never used.
  uint32_t a_off[NT][NF];  // LDS byte offset of this lane's A row at k = grp * 8
  int b_of[NF][NR];        // batch held by D register r (>= B: unused)
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int bb = 16 * f + 4 * (col & 3) + (col >> 2);
    if (bb >= B) bb = 16 * f;
#pragma unroll
    for (int t = 0; t < NT; ++t) a_off[t][f] = (uint32_t)(((t * B + bb) * row + grp * 8) * 2);
#pragma unroll
    for (int r = 0; r < NR; ++r) b_of[f][r] = 16 * f + 4 * r + grp;
  }
  const NibRegs nib = nib_regs();

  f32x4 acc[NTW][NF];
  auto zero_acc = [&]() {
#pragma unroll
    for (int u = 0; u < NTW; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[u][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  const uint32_t scl_lane = (uint32_t)col * SEG;
  auto compute = [&](const uint4 (&w)[CHK][NTW], int c) {
    if (q0 >= q1) return;  // empty quarter (uniform): nothing staged to read
    const int il = citem(c);
    const int cb = q0 + (c - il * cpi) * CHK;
    const uint8_t* const s_act_c = (const uint8_t*)s_act;
    // A K block past the quarter was loaded from a valid block (its load is
    // unconditional, see above).  Above 8 sequences the K splits leave such
    // slots in most chunks, and they are skipped: the branch is wave-uniform
    // and holds no memory load (measured on MI355X: the 8B O projection at
    // batch 32 43 -> 25 us, the whole 70B block at batch 32 875 -> 666 us).
    // Up to 8 sequences (where such slots are rare) the branch-free form
    // (weight 0) is kept: the branch cost 0.3-0.5 us on the 8B O and gate/up
    // projections at batch 1.
    constexpr bool kSkipPast = NR == 4;
#pragma unroll
    for (int i = 0; i < CHK; ++i) {
      const bool live = cb + i < q1;
      if constexpr (kSkipPast) {
        if (!live) continue;
      }
      const int kb = live ? cb + i : (q0 < q1 ? q0 : kb0);
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
          for (int u = 0; u < NTW; ++u) bw[u] = widen_word_fast(word_of(w[i][u], s), nib);
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int f = 0; f < NF; ++f) {
              const bf16x8 av = *(const bf16x8*)(s_act_c + a_off[t][f] + (kb - kb0) * 256 + s * 64);
#pragma unroll
              for (int u = 0; u < NTW; ++u) d[u][f] = mfma16(av, bw[u], d[u][f]);
            }
        }
        const int jl = (kb - kb0) * (128 / G) + gi;
#pragma unroll
        for (int u = 0; u < NTW; ++u) {
          const uint16_t* st = s_scl + ((size_t)((il * NTW + u) * nkb8 + (kb >> 3) - b80) * 16) * SEG +
                               (kb & 7) * (128 / G) + gi;
          // read unconditionally (kb is clamped into the staged range), then
          // select: no branch around the LDS read
          const float sv = half_bits_to_f32(st[scl_lane]);
          const float scale = live ? sv : 0.f;
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int r = 0; r < NR; ++r) {
              const int b = b_of[f][r] < B ? b_of[f][r] : 0;
              const float2 gs = s_gsum[(size_t)b * ngr + jl];
              acc[u][f][r] = fmaf(scale, remove_offset(d[u][f][r], gs), acc[u][f][r]);
            }
        }
      }
    }
  };

  auto part = [&](int slot, int w, int u, int f, int r) -> float& {
    return s_part[((((slot * NW + w) * NTW + u) * NF + f) * NR + r) * 64 + lane];
  };

  // end of an item: add the NW wave sums in LDS; one wave (rotating) keeps
  // the item's sums in LDS while the others go on streaming.  No global
  // memory access happens here: on this target stores count in vmcnt too.
  auto finish_item = [&](int item, int slot) {
#pragma unroll
    for (int u = 0; u < NTW; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int r = 0; r < NR; ++r) part(slot, wq, u, f, r) = acc[u][f][r];
    zero_acc();
    __syncthreads();
    if (wq != (item - it0) % NW) return;
#pragma unroll
    for (int u = 0; u < NTW; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          // fixed pairwise order over the NW wave sums
          float o;
          if constexpr (NW == 4) {
            o = (part(slot, 0, u, f, r) + part(slot, 1, u, f, r)) + (part(slot, 2, u, f, r) + part(slot, 3, u, f, r));
          } else {
            float v[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) v[w] = part(slot, w, u, f, r);
#pragma unroll
            for (int h = 1; h < NW; h <<= 1)
#pragma unroll
              for (int w = 0; w + h < NW; w += 2 * h) v[w] += v[w + h];
            o = v[0];
          }
          const int tok = b_of[f][r];
          if (tok < B) s_out[(((item - it0) * NTW + u) * B + tok) * 16 + col] = o;
        }
  };
  auto finish = [&](int c) {
    const int ci = citem(c);
    if (c + 1 == (ci + 1) * cpi) finish_item(it0 + ci, ci & 1);
  };

  // Prologue: the activation loads (when they fit in registers) go out
  // first, then the first weight chunk(s); staging then waits for the
  // activation only.  Both staging paths end with only weight loads in
  // flight.
  auto prologue = [&](auto two_chunks, auto maxp) {
    // passes held in registers: the smallest of 1, 2, 4 and MAXP that
    // covers the wave's passes, so that no load repeats a pass (such loads
    // still occupy the CU's vector-memory path, which bounds the prologue:
    // measured on MI355X, 8B block at batch 8 88 -> 84 us, 70B 191 -> 185)
    constexpr int MP = decltype(maxp)::value;
    // scales first (oldest loads: waiting for them does not wait for
    // weights), in four named registers, not an array (a conditionally
    // assigned register array is placed in scratch)
    static_assert(MAXS == 4, "four scale pieces per thread");
    // A wave whose threads are all past the last piece skips that load and
    // its store (wave-uniform branches): the repeated loads occupied the
    // CU's vector-memory path like any other (measured on MI355X, 8B at
    // batch 1: QKV 7.7 -> 7.1 us, down 11.7 -> 10.5; block at batch 8
    // 85 -> 83).  Threads of a live wave past the last piece load and
    // rewrite the last piece (clamped indices).
    const int wbase = wq * 64;
    const bool l0 = wbase < npieces, l1 = NTH + wbase < npieces, l2 = 2 * NTH + wbase < npieces,
               l3 = 3 * NTH + wbase < npieces;
    uint4 sr0 = uint4{0, 0, 0, 0}, sr1 = sr0, sr2 = sr0, sr3 = sr0;
    if (l0) sr0 = *scl_src(min(tid, npieces - 1));
    if (l1) sr1 = *scl_src(min(NTH + tid, npieces - 1));
    if (l2) sr2 = *scl_src(min(2 * NTH + tid, npieces - 1));
    if (l3) sr3 = *scl_src(min(3 * NTH + tid, npieces - 1));
    auto store_scales = [&]() {
      if (l0) ((uint4*)s_scl)[min(tid, npieces - 1)] = sr0;
      if (l1) ((uint4*)s_scl)[min(NTH + tid, npieces - 1)] = sr1;
      if (l2) ((uint4*)s_scl)[min(2 * NTH + tid, npieces - 1)] = sr2;
      if (l3) ((uint4*)s_scl)[min(3 * NTH + tid, npieces - 1)] = sr3;
    };
    if (npass <= MP) {
      // passes past npass repeat a valid one and are skipped; the mask is
      // opaque to the compiler so the unrolled loop keeps static register
      // indices (a bound it could see turns into a loop over a dynamically
      // indexed array in scratch)
      uint32_t live_pass = (1u << npass) - 1u;
      asm volatile("" : "+s"(live_pass));
      ActRegs r[MP];
#pragma unroll
      for (int p = 0; p < MP; ++p) act_load(min(p, npass - 1), r[p]);  // clamped; see above
      load_chunk(wA, 0);
      if constexpr (decltype(two_chunks)::value) load_chunk(wB, 1);
#pragma unroll
      for (int p = 0; p < MP; ++p) act_store(p, r[p], (live_pass >> p) & 1u);
      store_scales();
    } else {
      // MP passes per round trip (loads clamped, stores guarded)
      for (int p0 = 0; p0 < npass; p0 += MP) {
        ActRegs r[MP];
#pragma unroll
        for (int p = 0; p < MP; ++p) act_load(min(p0 + p, npass - 1), r[p]);
#pragma unroll
        for (int p = 0; p < MP; ++p) act_store(p0 + p, r[p], p0 + p < npass);
      }
      store_scales();
      load_chunk(wA, 0);
      if constexpr (decltype(two_chunks)::value) load_chunk(wB, 1);
    }
    // pieces beyond the registers (the planner avoids this; correct but slow)
    for (int q = MAXS * NTH + tid; q < npieces; q += NTH) ((uint4*)s_scl)[q] = *scl_src(q);
    zero_acc();
    __syncthreads();  // scales (and group sums of squares) of the whole workgroup
    // RMSNorm sums of squares of the rows, by wave 0 while the weights
    // stream (fixed butterfly order); read after the epilogue's barrier
    if constexpr (F32) {
      if (wq == 0) {
        for (int b = 0; b < B; ++b) {
          float t = 0.f;
          for (int g = lane; g < ngr; g += 64) t += s_sqg[(size_t)b * ngr + g];
          t = wave_sum(t);
          if (lane == 0) s_ss[b] = t;
        }
      }
    }
  };

  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, MAXP < 2 ? MAXP : 2>;
  using P4 = std::integral_constant<int, MAXP < 4 ? MAXP : 4>;
  using PM = std::integral_constant<int, MAXP>;
  auto run_prologue = [&](auto two_chunks) {
    if (npass <= 1) prologue(two_chunks, P1{});
    else if (npass <= 2) prologue(two_chunks, P2{});
    else if (npass <= 4 || MAXP == 4) prologue(two_chunks, P4{});
    else prologue(two_chunks, PM{});
  };
  if (nchunks == 1) {
    run_prologue(std::false_type{});
    compute(wA, 0);
    finish(0);
  } else {
    run_prologue(std::true_type{});
    // Main loop over chunk pairs with unconditional loads; the last one to
    // three chunks are peeled.
    int c = 0;
    for (; c + 3 < nchunks; c += 2) {
      compute(wA, c);
      load_chunk(wA, c + 2);
      finish(c);
      compute(wB, c + 1);
      load_chunk(wB, c + 3);
      finish(c + 1);
    }
    compute(wA, c);
    if (c + 2 < nchunks) load_chunk(wA, c + 2);
    finish(c);
    compute(wB, c + 1);
    finish(c + 1);
    if (c + 2 < nchunks) {
      compute(wA, c + 2);
      finish(c + 2);
    }
  }
  __syncthreads();

  // ---- epilogue and write-out of the workgroup's items
  const int nout = (it1 - it0) * B * 16;
  for (int idx = tid; idx < nout; idx += NTH) {
    const int il = dbr.div(idx), rem = idx - il * B * 16, tok = rem >> 4, cc = rem & 15;
    const int n = (it0 + il) * 16 + cc;  // physical row (non-pair) / logical column (pair)
    const float o = s_out[((il * NTW) * B + tok) * 16 + cc];
    if constexpr (EPI == kEpiPartial) {
      a.out[((size_t)split * a.B + b0 + tok) * a.N + n] = o;
    } else if constexpr (EPI == kEpiRms) {
      a.out[(size_t)(b0 + tok) * a.N + n] = o * (1.0f / sqrtf(s_ss[tok] / (float)a.K + a.eps));
    } else if constexpr (EPI == kEpiResid) {
      const float rv = idx == tid ? resid_pf : a.resid[(size_t)(b0 + tok) * a.N + n];
      a.out[(size_t)(b0 + tok) * a.N + n] = rv + o;
    } else {  // kEpiSwiglu: u = 0 gate rows, u = 1 up rows of logical column n
      const float invr = 1.0f / sqrtf(s_ss[tok] / (float)a.K + a.eps);
      const float g = o * invr, up = s_out[((il * NTW + PAIR) * B + tok) * 16 + cc] * invr;
      a.out_bf16[(size_t)(b0 + tok) * a.inter + n] = f32_to_bf16_bits(g / (1.0f + expf(-g)) * up);
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

// rows of the largest batch tile
static int tile_rows(const GemmArgs& a) {
  const int nt = a.ntiles > 1 ? a.ntiles : 1;
  return (a.B + nt - 1) / nt;
}

size_t gemm_lds_bytes(const GemmArgs& a, int nterms, int G, bool pair) {
  const int krange = a.kb_per_wg;
  const int bt = tile_rows(a);
  const int nf = bt <= 16 ? 1 : 2;
  const int nr = bt <= 4 ? 1 : bt <= 8 ? 2 : 4;
  const int items_wg = (a.items + a.wgs_per_split - 1) / a.wgs_per_split;
  const int nkb8 = (krange + 7) / 8 + 1;  // a K range not aligned to 8 blocks spans one more
  return gemm_lds_layout(nterms, bt, krange, G, pair ? 2 : 1, nf * nr, items_wg, nkb8, a.nw).total;
}

static size_t plan_lds(const GemmPlan2& p, int B, int G, int nterms, bool pair) {
  GemmArgs a{};
  a.B = B;
  a.kb_per_wg = p.kb_per_wg;
  a.items = p.items;
  a.wgs_per_split = p.wgs_per_split;
  a.nw = p.nw;
  return gemm_lds_bytes(a, nterms, G, pair);
}

// Items per workgroup for a plan whose splits and waves are set: spread the
// items evenly over `occ` workgroups per CU, fewer per workgroup while the
// LDS or the scale registers do not hold them.
static void plan_items(GemmPlan2& p, int B, int G, int nterms, bool pair, int occ, int cus) {
  const int target = (occ * cus + p.splits - 1) / p.splits;
  int per = (p.items + target - 1) / target;
  if (per < 1) per = 1;
  // scale staging: at most 4 16-byte pieces per thread (registers)
  const int nkb8 = (p.kb_per_wg + 7) / 8 + 1;
  auto pieces = [&](int ipw) { return (long)ipw * (pair ? 2 : 1) * nkb8 * 16 * (128 / G); };
  for (;;) {
    p.wgs_per_split = (p.items + per - 1) / per;
    if (per == 1 || (plan_lds(p, B, G, nterms, pair) <= (size_t)kLdsMax && pieces(per) <= 4L * 64 * p.nw)) break;
    --per;
  }
}

// Plan of one batch tile of B rows on `cus` CUs.
static GemmPlan2 plan_tile(int N, int K, int G, int B, int nterms, int epi, int cus) {
  GemmPlan2 p;
  const int KB = K / 128;
  const bool pair = epi == kEpiSwiglu;
  const int items = pair ? N / 32 : N / 16;
  // K splits: only kEpiPartial may split; split until the activation range
  // fits the LDS budget
  p.splits = 1;
  if (epi == kEpiPartial) {
    while (p.splits < KB && (long)nterms * B * ((KB + p.splits - 1) / p.splits) * 256 > kLdsActBudget) ++p.splits;
  }
  p.kb_per_wg = (KB + p.splits - 1) / p.splits;
  p.splits = (KB + p.kb_per_wg - 1) / p.kb_per_wg;
  p.items = items;
  // Above 4 sequences every workgroup stages several activation rows, so
  // the LDS holds one workgroup per CU.  Sixteen waves then share that one
  // staged copy (four per SIMD, which hides the matrix-core, LDS and
  // dequantization latencies of one another), each owning at least one K
  // block of every item (a 16-block range: measured on MI355X, 8B down
  // projection at batch 8 18.7 -> 16.8 us, 8B batch 16 down 40 -> 35 us).
  // One workgroup per CU: the items are spread over min(items, CUs /
  // splits) workgroups (the kernel gives each an even share, so item counts
  // differ by at most one), more while a share does not fit the LDS.
  // Below 5 sequences the same shape wins for large projections, where the
  // 4-wave workgroups staging B activation rows each leave one or two
  // workgroups per CU (measured on MI355X, 70B: O at batch 4 25.8 -> 15.6
  // us, gate/up at batch 1 53 -> 45 us, down at batch 2 45 -> 28 us, QKV at
  // batch 1 14.3 -> 13.4 us), but not for small ones at small batch (8B O
  // at batch 2 6.4 -> 7.9 us): from batch 4 always, below with at least
  // 128 KiB of weights per CU (and K >= 64 blocks at batch 1).
  const long wcu = (long)N * K / 2 / cus;
  const bool deep = B >= 4 || (wcu >= (128L << 10) && (B >= 2 || KB >= 64));
  // A plan that needs more workgroups than CUs (the items of a share do not
  // fit the LDS) runs a second, partial round; K splits beyond the LDS
  // minimum (kEpiPartial) shrink the staged range until one round holds
  // the items (measured on MI355X: 70B down at batch 8 in 8 instead of 7
  // splits 57 -> 35 us, at batch 16 in two 8-row tiles 92 -> 56 us).
  // Without such a split the first plan that fits is kept.
  if (deep && p.kb_per_wg >= 16) {
    GemmPlan2 first;
    bool have = false;
    for (GemmPlan2 sp = p;;) {
      GemmPlan2 q = sp;
      q.nw = 16;
      plan_items(q, B, G, nterms, pair, 1, cus);
      const int even = std::min(items, std::max(1, cus / q.splits));
      if (even > q.wgs_per_split) {
        GemmPlan2 r = q;
        r.wgs_per_split = even;
        if (plan_lds(r, B, G, nterms, pair) <= plan_lds(q, B, G, nterms, pair)) q = r;
      }
      if (plan_lds(q, B, G, nterms, pair) <= (size_t)kLdsMax) {
        if (q.splits * q.wgs_per_split <= cus) return q;
        if (!have) first = q, have = true;
      }
      if (epi != kEpiPartial) break;
      int ns = sp.splits + 1, kb = 0;
      while (ns <= KB && (kb = (KB + ns - 1) / ns) == sp.kb_per_wg) ++ns;
      if (ns > KB || kb < 16) break;
      sp.kb_per_wg = kb;
      sp.splits = (KB + kb - 1) / kb;
    }
    if (have) return first;
  }
  // Waves per workgroup: when there are no more items than CUs and K is
  // long, one workgroup per item leaves each CU with few loads in flight, so
  // the item's K range is shared by more waves (measured on MI355X: faster
  // for the 8B down projection, K = 14336; slower for K = 4096).  Sixteen
  // waves (chunks of two K blocks) beat eight there: 8B down at batch 4
  // 15.8 -> 14.5 us, batch 1 equal.
  p.nw = 4;
  if (p.splits == 1 && (long)items * 100 <= (long)cus * FUTX_GEMM_WIDE_PCT && KB >= 64) p.nw = FUTX_GEMM_WIDE_NW;
  // Workgroups per CU aimed at: three for up to 4 sequences; one above,
  // where every workgroup stages B activation rows, so fewer workgroups
  // with more items each stage less (measured on MI355X at batch 8: the 8B
  // gate/up projection 32.1 -> 23.4 us; at batch 1 three per CU is best).
  plan_items(p, B, G, nterms, pair, B <= 4 ? FUTX_GEMM_OCC : FUTX_GEMM_OCC_BATCH, cus);
  return p;
}

static GemmPlan2 plan_tiled(int N, int K, int G, int B, int nterms, int epi, int nt) {
  const int cus = device_cu_count();
  GemmPlan2 p = plan_tile(N, K, G, (B + nt - 1) / nt, nterms, epi, std::max(1, cus / nt));
  p.ntiles = nt;
  return p;
}

// Whether a plan of a fused epilogue applies.
static bool tile_fits(const GemmPlan2& p, int B, int G, int nterms, int epi) {
  B = (B + p.ntiles - 1) / p.ntiles;  // rows of a tile
  // a 16-wave plan in more than one round: the K split (one round) is
  // faster (measured on MI355X, 70B down at batch 8 57 -> 35 us)
  if (p.nw == 16 && (long)p.ntiles * p.splits * p.wgs_per_split > device_cu_count()) return false;
  // Above 4 sequences a fused epilogue is taken only with 16 waves: a
  // 4-wave workgroup that fills the LDS alone (one wave per SIMD) is slower
  // than the 16-wave K split with its finishing kernels (measured on MI355X:
  // 70B gate/up at batch 8 95 -> 67 us, 8B gate/up at batch 16 50 -> 40 us).
  if (B >= FUTX_GEMM_DEEP_MIN_B && p.nw != 16) return false;
  return plan_lds(p, B, G, nterms, epi == kEpiSwiglu) <= (size_t)kLdsMax;
}

// Batch tiles above 8 sequences.  Every tile streams all the weights (from
// the L2 of its XCD after the first), so tiling trades weight-block slots
// for a smaller staged activation: fewer K splits and empty chunk slots.
// The plans compared here have one workgroup per CU; the estimate is the
// critical path per CU in weight-block slots (rounds x items per workgroup x
// slots per item, empty ones included: their loads are issued), plus a
// fixed charge for the finishing kernels of a K split; ties go to fewer
// tiles.  Measured on MI355X against one tile: 8B at batch 16 in 8-row
// tiles 152 -> 113 us per block; 70B down at batch 16 78 -> 56 us, while
// 70B O and gate/up at batch 16 stay in one tile (31.6 vs 38.6 and 119.7
// vs 146.6 us in two), as the estimate has it.
constexpr double kSplitCharge = 32.0;

static double plan_cost(const GemmPlan2& p, int B, bool pair) {
  const int bt = (B + p.ntiles - 1) / p.ntiles;
  const int ntw = pair ? 2 : 1;
  const long ipw = (p.items + p.wgs_per_split - 1) / p.wgs_per_split;
  const int kbq = (p.kb_per_wg + p.nw - 1) / p.nw;
  const int chk = p.nw == 16 ? 2 : (pair || bt > 16) ? 4 : 8;
  const long slots = (long)(kbq + chk - 1) / chk * chk * p.nw;
  const long cus = device_cu_count();
  const long rounds = ((long)p.ntiles * p.splits * p.wgs_per_split + cus - 1) / cus;
  return (double)(rounds * ipw * ntw * slots);
}

// Tile counts compared: tiles of at most 16 and at most 8 rows (one tile up
// to 8 sequences).  Tiles of more than 16 rows are not used: with two
// matrix-core fragments per weight block they measured slower than 8-row
// tiles for every projection (8B at batch 32: 247 vs 162 us per block).
static int tile_counts(int B, int (&nt)[3]) {
  int n = 0;
  for (int rows : {16, 8}) {
    const int t = (B + rows - 1) / rows;
    if (n == 0 || t != nt[n - 1]) nt[n++] = t;
  }
  return n;
}

static GemmPlan2 best_partial(int N, int K, int G, int B, int nterms, double* cost) {
  int nt[3];
  const int n = tile_counts(B, nt);
  GemmPlan2 best;
  double bc = 0.0;
  for (int i = 0; i < n; ++i) {
    const GemmPlan2 q = plan_tiled(N, K, G, B, nterms, kEpiPartial, nt[i]);
    const double c = plan_cost(q, B, false) + kSplitCharge;
    if (i == 0 || c < bc) best = q, bc = c;
  }
  if (cost) *cost = bc;
  return best;
}

// Plan of an epilogue: fused (one kernel) or, when that does not fit or is
// estimated slower, the K-split partial plan whose sums separate kernels
// finish.  Up to 8 sequences: one tile, fused whenever it fits.
static GemmPlan2 choose(int N, int K, int G, int B, int nterms, int epi, bool* fused) {
  *fused = false;
  if (epi == kEpiPartial) return best_partial(N, K, G, B, nterms, nullptr);
  int nt[3];
  const int n = tile_counts(B, nt);
  GemmPlan2 best;
  double bc = 0.0;
  for (int i = 0; i < n; ++i) {
    const GemmPlan2 f = plan_tiled(N, K, G, B, nterms, epi, nt[i]);
    if (!tile_fits(f, B, G, nterms, epi)) continue;
    const double c = plan_cost(f, B, epi == kEpiSwiglu);
    if (!*fused || c < bc) best = f, bc = c, *fused = true;
  }
  if (*fused && B <= 8) return best;
  double pc;
  const GemmPlan2 q = best_partial(N, K, G, B, nterms, &pc);
  // Up to 8 sequences, a K split that leaves 16-wave chunks half empty (one
  // K block per wave) loses to the fused plan in two batch tiles when that
  // fits (measured on MI355X, 70B O at batch 8 23.2 -> 20.5 us, batch 5
  // 22.6 -> 18.9); with full chunks the K split stays (8B down, 70B gate/up
  // and down were slower in two tiles).
  if (!*fused && B <= 8 && B >= 2 && q.nw == 16 && (q.kb_per_wg + 15) / 16 < 2) {
    const GemmPlan2 f = plan_tiled(N, K, G, B, nterms, epi, 2);
    if (tile_fits(f, B, G, nterms, epi)) {
      *fused = true;
      return f;
    }
  }
  if (!*fused || pc < bc) {
    *fused = false;
    return q;
  }
  return best;
}

GemmPlan2 plan_gemm(int N, int K, int G, int B, int nterms, int epi) {
  bool fused;
  return choose(N, K, G, B, nterms, epi, &fused);
}

bool gemm_fits(int N, int K, int G, int B, int nterms, int epi) {
  bool fused;
  choose(N, K, G, B, nterms, epi, &fused);
  return fused;
}

hipError_t launch_int4_gemm(GemmArgs a, int G, int nterms, bool act_f32, int epi, hipStream_t st) {
  const bool pair = epi == kEpiSwiglu;
  const int ntl = a.ntiles > 1 ? a.ntiles : 1, bt = tile_rows(a);
  const int nwg = a.splits * a.wgs_per_split;
  const dim3 grid(ntl > 1 ? (nwg + 7) / 8 * 8 * ntl : nwg), block(64 * a.nw);
  // batch tiles of at most 16 rows (one matrix-core fragment; the planner
  // makes no larger ones)
  if (ntl > a.B || bt > 16) return hipErrorInvalidValue;
  if (a.splits != 1 && epi != kEpiPartial) return hipErrorInvalidValue;
  if (a.nw != 4 && a.nw != FUTX_GEMM_WIDE_NW && a.nw != 16) return hipErrorInvalidValue;
  const size_t lds = gemm_lds_bytes(a, nterms, G, pair);
  if (lds > (size_t)kLdsMax) return hipErrorInvalidValue;
#define FUTX_G(GG, NF, NR, NT, F32, EPI, PR) \
  do {                                   \
    auto k_ = a.nw == 4 ? int4_gemm_kernel<GG, NF, NR, NT, F32, EPI, PR, 4> \
              : a.nw == 16 ? int4_gemm_kernel<GG, NF, NR, NT, F32, EPI, PR, 16> \
                           : int4_gemm_kernel<GG, NF, NR, NT, F32, EPI, PR, FUTX_GEMM_WIDE_NW>; \
    if (lds > 64 * 1024) {                                                  \
      const hipError_t e_ = hipFuncSetAttribute((const void*)k_, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
      if (e_ != hipSuccess) return e_;                                      \
    }                                                                       \
    k_<<<grid, block, lds, st>>>(a); \
  } while (0)
#define FUTX_NF(GG, NT, F32, EPI, PR) \
  do {                                  \
    if (bt <= 4) FUTX_G(GG, 1, 1, NT, F32, EPI, PR);                   \
    else if (bt <= 8) FUTX_G(GG, 1, 2, NT, F32, EPI, PR);              \
    else FUTX_G(GG, 1, 4, NT, F32, EPI, PR);                           \
  } while (0)
#define FUTX_GRP(NT, F32, EPI, PR)                                        \
  do {                                                                     \
    if (G == 128) FUTX_NF(128, NT, F32, EPI, PR); else FUTX_NF(64, NT, F32, EPI, PR); \
  } while (0)
  switch (epi) {
    case kEpiPartial:
      if (nterms == FUTX_O_TERMS) FUTX_GRP(FUTX_O_TERMS, false, kEpiPartial, 0);
      else if (act_f32) FUTX_GRP(1, true, kEpiPartial, 0);
      else FUTX_GRP(1, false, kEpiPartial, 0);
      break;
    case kEpiRms: FUTX_GRP(1, true, kEpiRms, 0); break;
    case kEpiResid:
      if (nterms == FUTX_O_TERMS) FUTX_GRP(FUTX_O_TERMS, false, kEpiResid, 0); else FUTX_GRP(1, false, kEpiResid, 0);
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
