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

hipError_t launch_prep_act(const float* x, int B, int H, float eps, uint16_t* act, float* invr,
                           hipStream_t st);
hipError_t launch_gsum(const uint16_t* act, int B, int K, int G, float2* gsum, hipStream_t st);
hipError_t launch_reduce(const float* part, int S, int B, int N, const float* rowscale,
                         const float* resid, float* out, int gateup_inter, hipStream_t st);
hipError_t launch_swiglu(const float* part, int S, int B, int I, int G, const float* invr,
                         uint16_t* act, float2* gsum, hipStream_t st);
hipError_t launch_kv_append(const float* k, const float* v, const int32_t* positions,
                            const int32_t* slots, int n, uint32_t flags, int D, int hb,
                            float theta, const KVPtrs& kv, hipStream_t st);
// The attention part of the decode block before the merge (new-token
// append, rotated queries, split attention, four splits merged per
// workgroup): reads the QKV projection qkv [B][(nq + 2 nkv) D] fp32, writes
// wpart [B][nq][ceil(nsplit / 4)][D + 2]; finish with launch_attn_merge
// on a plan of 4 * chunk tokens and ceil(nsplit / 4) splits.
hipError_t launch_attn_decode(const float* qkv, const int32_t* cached_lens, const int32_t* block_table,
                              int mpps, int B, int nq, int D, const AttnPlan& plan, int hb, float theta,
                              const KVPtrs& kv, float* wpart, hipStream_t st);
// q: rotated queries [B][nq][D], fp32 (q_f32) or bf16
hipError_t launch_attention(const void* q, bool q_f32, const int32_t* lens, int len_add,
                            const int32_t* block_table, int mpps, int B, int nq, int D,
                            const AttnPlan& plan, const KVPtrsConst& kv, float* apart,
                            hipStream_t st);
// out_bf16: FUTX_O_TERMS bf16 terms of o (gemm.h), term t at out_bf16 + t * term_stride
hipError_t launch_attn_merge(const float* apart, const int32_t* lens, int len_add, int B, int nq,
                             int D, const AttnPlan& plan, int hb, float* out_f32,
                             uint16_t* out_bf16, size_t term_stride, hipStream_t st);

}  // namespace futx
