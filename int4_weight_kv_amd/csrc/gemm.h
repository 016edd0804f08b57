// INT4 projection GEMM (gemm.hip): arguments, epilogues, planning.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// bf16 terms of the O projection operand: the attention output o enters
// the matrix cores as hi + lo with hi = bf16(o), lo = bf16(o - hi), so
// |o - hi - lo| <= 2^-18 |o| (three terms would carry it to fp32 accuracy;
// measured on MI355X, two terms halve the O projection at batch 8 and above,
// with every block parity case still within tolerance)
#ifndef FUTX_O_TERMS
#define FUTX_O_TERMS 2
#endif

namespace futx {

// LDS budget of a workgroup's staged activation range (two workgroups per
// CU fit), and the largest LDS allocation of one workgroup (gfx950: 160 KB).
constexpr long kLdsActBudget = 72 * 1024;
constexpr long kLdsMax = 160 * 1024;

// Epilogues of int4_gemm_kernel.
constexpr int kEpiPartial = 0;  // out[split][b][n] = partial sum (fp32, physical rows)
constexpr int kEpiRms = 1;      // out[b][n] = sum / r_b, r_b = RMS of the fp32 activation row
constexpr int kEpiResid = 2;    // out[b][n] = resid[b][n] + sum
constexpr int kEpiSwiglu = 3;   // out_bf16[b][c] = bf16(silu(g / r_b) * u / r_b) for gate/up tile pairs

struct GemmArgs {
  const uint4* w;        // packed weights (layout.h)
  const uint16_t* sc;    // fp16 group scales [N][K / G]
  const void* act;       // activations: bf16 [terms][B][K] or fp32 [B][K]
  size_t term_stride;    // elements between bf16 terms
  int N, K, B;
  int splits;            // K splits
  int kb_per_wg;         // K blocks (128 inputs) per split
  int items;             // 16-row tiles (gate/up pairs for kEpiSwiglu)
  int wgs_per_split;     // workgroups per split, each with a run of items
  int nw;                // waves per workgroup
  int ntiles;            // batch tiles (rows split evenly; 0 or 1: one tile)
  float eps;             // RMSNorm epsilon
  const float* resid;    // kEpiResid
  float* out;            // kEpiPartial / kEpiRms / kEpiResid
  uint16_t* out_bf16;    // kEpiSwiglu
  int inter;             // kEpiSwiglu: row stride (intermediate size) of out_bf16
};

// LDS carve of int4_gemm_kernel (byte offsets, each 16-byte aligned).
struct GemmLds {
  size_t act, gsum, sqg, part, ss, out, scl, total;
};
__host__ __device__ inline GemmLds gemm_lds_layout(int nterms, int B, int krange, int G, int ntw, int nfr,
                                                   int items_wg, int nkb8, int nw) {
  auto up = [](size_t x) { return (x + 15) & ~(size_t)15; };
  const int ngr = krange * 128 / G;
  GemmLds l;
  l.act = 0;
  l.gsum = up(l.act + (size_t)nterms * B * (krange * 128 + 8) * 2);
  l.sqg = up(l.gsum + (size_t)B * ngr * 8);
  l.part = up(l.sqg + (size_t)B * ngr * 4);
  l.ss = up(l.part + (size_t)2 * nw * ntw * nfr * 64 * 4);
  l.out = up(l.ss + (size_t)B * 4);
  l.scl = up(l.out + (size_t)items_wg * ntw * B * 16 * 4);
  l.total = up(l.scl + (size_t)items_wg * ntw * nkb8 * 16 * (8 * 128 / G) * 2);
  return l;
}

struct GemmPlan2 {
  int nw = 4;  // waves per workgroup (4, 8 or 16), each owning 1 / nw of the K range
  int splits = 1;
  int kb_per_wg = 1;
  int items = 1;
  int wgs_per_split = 1;
  int ntiles = 1;  // batch tiles, each planned as its own batch on CUs / ntiles
};

// Work plan: K splits (only kEpiPartial splits K, until the activation
// range fits the LDS budget) and workgroups per split.
GemmPlan2 plan_gemm(int N, int K, int G, int B, int nterms, int epi);
// Whether the single-split plan of an epilogue fits in LDS (otherwise the
// caller splits K with kEpiPartial and finishes with separate kernels).
bool gemm_fits(int N, int K, int G, int B, int nterms, int epi);
int device_cu_count();
void apply_plan(GemmArgs& a, const GemmPlan2& p);
hipError_t launch_int4_gemm(GemmArgs a, int G, int nterms, bool act_f32, int epi, hipStream_t st);

inline void apply_plan(GemmArgs& a, const GemmPlan2& p) {
  a.splits = p.splits;
  a.kb_per_wg = p.kb_per_wg;
  a.items = p.items;
  a.wgs_per_split = p.wgs_per_split;
  a.nw = p.nw;
  a.ntiles = p.ntiles;
}

}  // namespace futx
