// Launchers of the gfx950 kernels (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace futx {

struct KVPtrs {
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint16_t* k_scales;
  uint16_t* v_scales;
  int nkv;
};

struct KVPtrsConst {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint16_t* k_scales;
  const uint16_t* v_scales;
  int nkv;
};

struct AttnPlan {
  int chunk = 64;  // tokens per split (multiple of the page size)
  int nsplit = 1;  // splits per sequence for the largest context
};

AttnPlan attn_plan(int B, int nkv, int max_context);
// an upper bound of attn_plan(B, nkv, c).nsplit over c <= max_context,
// non-decreasing in max_context (sizes the workspace)
int attn_nsplit_bound(int B, int nkv, int max_context);

// Arguments of the decode attention kernel (kernels.hip).
struct AttnArgs {
  const float* qkv;            // [B][(nq + 2 nkv) D] fp32 QKV projection (before RoPE)
  const int32_t* cached_lens;  // [B] new token's position
  const int32_t* block_table;  // [B][mpps]
  int mpps;                    // block table row length (pages)
  int nq;                      // query heads
  int chunk;                   // tokens per split (set by launch_attn_decode)
  int nwg;                     // workgroups per sequence (4 splits each; set by launch_attn_decode)
  int hb;                      // Hadamard block
  int tmax;                    // largest L_b + 1 the plan covers
  float theta;                 // RoPE base
  float scale;                 // 1 / sqrt(D) (set by launch_attn_decode)
  double inv_freq[64];         // RoPE inverse frequencies theta^(-2i/D), i < D/2 (set by launch_attn_decode)
  KVPtrs kv;
  float* wpart;                // [B][nq][nwg][D + 2] workgroup partials
  float* out_f32;              // [B][nq][D] attention output, or null
  uint16_t* out_bf16;          // FUTX_O_TERMS bf16 terms of [B][nq D] (O projection operand), or null
  size_t term_stride;          // elements between the bf16 terms
};

// RMS statistics of fp32 rows x[B][H] (H a multiple of 128): invr[b] =
// 1 / sqrt(mean(x_b^2) + eps), and, when act is not null, the rows rounded
// to bf16 in act[B][H].
hipError_t launch_prep_act(const float* x, int B, int H, float eps, uint16_t* act, float* invr,
                           hipStream_t st);
hipError_t launch_reduce(const float* part, int S, int B, int N, const float* rowscale,
                         const float* resid, float* out, int gateup_inter, hipStream_t st);
hipError_t launch_swiglu(const float* part, int S, int B, int I, const float* invr, uint16_t* act,
                         hipStream_t st);
hipError_t launch_kv_append(const float* k, const float* v, const int32_t* positions,
                            const int32_t* slots, int n, uint32_t flags, int D, int hb,
                            float theta, const KVPtrs& kv, hipStream_t st);
// The attention part of the decode block: new-token append, rotated
// queries, split attention (attn_decode_kernel), then, when the plan has
// more than one workgroup per sequence, the merge of the workgroup partials
// with the inverse rotation (attn_merge_kernel).
hipError_t launch_attn_decode(AttnArgs a, int B, int D, const AttnPlan& plan, hipStream_t st);

}  // namespace futx
