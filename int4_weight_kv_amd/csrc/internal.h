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

}  // namespace futx
