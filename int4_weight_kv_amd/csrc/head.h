// Embedding and LM head of the full decode step (head.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace futx {

// LM head workspace: bf16 input rows, 1/r, fp32 partial sums of the K splits
// (for at most 16 rows at a time), top-1 keys.
struct HeadWs {
  uint16_t* u;
  float* invr;
  float* part;
  unsigned long long* keys;
  size_t bytes;
};
HeadWs head_ws(int hidden, int vocab, int max_batch, char* base);  // base == nullptr: sizes only
bool head_shape_ok(int hidden);                                    // hidden a multiple of 256

hipError_t launch_embed(const uint16_t* table, const int32_t* tokens, int vocab, int H, int B, float* x,
                        hipStream_t st);
hipError_t launch_lm_head(const uint16_t* w, const float* x, int B, int H, int V, float eps, const HeadWs& ws,
                          float* logits, int32_t* top1, hipStream_t st);

}  // namespace futx
