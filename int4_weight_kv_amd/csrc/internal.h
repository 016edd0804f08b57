// Host-side helpers shared by the C-ABI translation units.
#pragma once

#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>

#include "futx.h"
#include "layout.h"

namespace futx {

// Records a message for futx_last_error() and returns `status`.
futx_status fail(futx_status status, const char* fmt, ...);
void clear_error();

struct ProjShape {
  int n;  // output rows
  int k;  // inputs
};

inline ProjShape proj_shape(const futx_dims& d, futx_proj p) {
  switch (p) {
    case FUTX_PROJ_QKV: return {(d.n_heads + 2 * d.n_kv_heads) * d.head_dim, d.hidden};
    case FUTX_PROJ_O: return {d.hidden, d.n_heads * d.head_dim};
    case FUTX_PROJ_GATEUP: return {2 * d.intermediate, d.hidden};
    case FUTX_PROJ_DOWN: return {d.hidden, d.intermediate};
  }
  return {0, 0};
}

// Validates the block shape; returns FUTX_OK or an error (message recorded).
futx_status check_dims(const futx_dims* d);
futx_status check_proj(futx_proj p);

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace bytes futx_decode_block carves for exactly `batch` sequences and
// `max_context` (dims already checked).
size_t decode_workspace_bytes(const futx_dims& d, int batch, int max_context);

// futx_decode_block (stage < 0) or one of its stages, with a given
// workspace; validates every argument.
futx_status decode_block_impl(const futx_dims* dims, const futx_block_weights* w, int32_t batch, float* x,
                              const int32_t* cached_lens, const int32_t* block_table, int32_t max_pages_per_seq,
                              int32_t max_context, const futx_kv_cache* cache, void* workspace,
                              size_t workspace_bytes, void* stream, int stage);

}  // namespace futx
