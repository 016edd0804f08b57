// C-ABI entry points of libfutx.so (declared in include/futx.h): argument
// validation, workspace carving and the launch order of the decode block.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <vector>

#include "gemm.h"
#include "head.h"
#include "internal.h"
#include "kernels.h"

namespace futx {

futx_status pack_host(const futx_dims* dims, futx_proj proj, const float* w, const float* gain,
                      void* packed, void* scales);
futx_status pack_codes_host(const futx_dims* dims, futx_proj proj, const uint8_t* canon,
                            const uint16_t* canon_scales, void* packed, void* scales);
futx_status unpack_host(const futx_dims* dims, futx_proj proj, const void* packed,
                        const void* scales, uint8_t* canon, uint16_t* canon_scales);
futx_status fold_head_host(int32_t vocab, int32_t hidden, const uint16_t* w, const float* gain,
                           uint16_t* out);

static thread_local char g_err[512];

futx_status fail(futx_status status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_err[0] = 0; }

static futx_status hip_fail(hipError_t e, const char* what) {
  return fail(FUTX_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define FUTX_HIP(call, what)                      \
  do {                                            \
    hipError_t e_ = (call);                       \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

static bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

futx_status check_dims(const futx_dims* d) {
  if (!d) return fail(FUTX_E_ARG, "dims is NULL");
  if (d->hidden <= 0 || d->n_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 ||
      d->intermediate <= 0 || d->w_group <= 0 || d->had_block <= 0 || d->page_size <= 0)
    return fail(FUTX_E_ARG, "dims: every size must be positive");
  if (!(d->rms_eps >= 0.f) || !(d->rope_theta > 0.f)) return fail(FUTX_E_ARG, "dims: bad eps or theta");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(FUTX_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d->w_group != 64 && d->w_group != 128) return fail(FUTX_E_UNSUPPORTED, "w_group must be 64 or 128");
  if (!pow2(d->had_block) || d->had_block > 64 || d->had_block < 2 || d->head_dim % d->had_block)
    return fail(FUTX_E_UNSUPPORTED, "had_block must be a power of two <= 64 dividing head_dim");
  if (d->page_size != kPageSize) return fail(FUTX_E_UNSUPPORTED, "page_size must be 64");
  if (d->n_heads % d->n_kv_heads || d->n_heads / d->n_kv_heads > 16)
    return fail(FUTX_E_UNSUPPORTED, "n_heads must be a multiple of n_kv_heads with at most 16 per group");
  if (d->head_dim % d->w_group) return fail(FUTX_E_UNSUPPORTED, "head_dim must be a multiple of w_group");
  const int ks[3] = {d->hidden, d->n_heads * d->head_dim, d->intermediate};
  for (int k : ks)
    if (k % kTileK || k % (2 * d->w_group))
      return fail(FUTX_E_UNSUPPORTED, "projection inputs must be multiples of 128 and of 2 * w_group");
  if (d->hidden % kTileN || d->intermediate % kTileN) return fail(FUTX_E_UNSUPPORTED, "bad row count");

  return FUTX_OK;
}

futx_status check_proj(futx_proj p) {
  if (p < FUTX_PROJ_QKV || p > FUTX_PROJ_DOWN) return fail(FUTX_E_ARG, "unknown projection %d", (int)p);
  return FUTX_OK;
}

// ---------------------------------------------------------------- workspace

struct Ws {
  uint16_t* act;   // 3 x [32][Kmax] bf16 (GEMM operand; FUTX_O_TERMS terms for the O projection)
  float* invr;     // [32]
  float* invr2;    // [32]
  float* part;     // split-K partials
  float* qkv;      // [B][Nqkv]
  float* apart;    // [B][nq][workgroups per sequence][D + 2] attention partials
  float* h;        // [B][H]
  size_t bytes;
};

static int kmax(const futx_dims& d) {
  int k = d.hidden;
  if (d.n_heads * d.head_dim > k) k = d.n_heads * d.head_dim;
  if (d.intermediate > k) k = d.intermediate;
  return k;
}

static size_t part_floats(const futx_dims& d, int B) {
  size_t m = 0;
  for (int p = 0; p < 4; ++p) {
    ProjShape s = proj_shape(d, (futx_proj)p);
    GemmPlan2 g = plan_gemm(s.n, s.k, d.w_group, B, p == FUTX_PROJ_O ? FUTX_O_TERMS : 1, kEpiPartial);
    size_t v = (size_t)g.splits * B * s.n;
    if (v > m) m = v;
  }
  return m;
}

static Ws carve(const futx_dims& d, int B, int max_ctx, char* base) {
  Ws w{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + at : nullptr;
    at += round_up(bytes, 256);
    return p;
  };
  const int K = kmax(d);
  const int D = d.head_dim, nq = d.n_heads;
  const int nqkv = (d.n_heads + 2 * d.n_kv_heads) * D;
  // attention workgroups per sequence, for any context up to max_ctx
  const int nwg = (attn_nsplit_bound(B, d.n_kv_heads, max_ctx) + 3) / 4;
  w.act = (uint16_t*)take((size_t)3 * kMaxBatch * K * 2);
  w.invr = (float*)take(kMaxBatch * 4);
  w.invr2 = (float*)take(kMaxBatch * 4);
  w.part = (float*)take(part_floats(d, B) * 4);
  w.qkv = (float*)take((size_t)B * nqkv * 4);
  w.apart = (float*)take((size_t)B * nq * nwg * (D + 2) * 4);
  w.h = (float*)take((size_t)B * d.hidden * 4);
  w.bytes = at;
  return w;
}

static KVPtrs kv_ptrs(const futx_kv_cache* c, int nkv) {
  return KVPtrs{(uint8_t*)c->k_codes, (uint8_t*)c->v_codes, (uint16_t*)c->k_scales,
                (uint16_t*)c->v_scales, nkv};
}

static futx_status check_cache(const futx_kv_cache* c) {
  if (!c || !c->k_codes || !c->v_codes || !c->k_scales || !c->v_scales || c->num_pages <= 0)
    return fail(FUTX_E_ARG, "kv cache: null pointer or no pages");
  return FUTX_OK;
}

static futx_status check_qweight(const futx_qweight* q, const char* name) {
  if (!q || !q->packed || !q->scales) return fail(FUTX_E_ARG, "weights %s: null pointer", name);
  if (((uintptr_t)q->packed | (uintptr_t)q->scales) & 15)
    return fail(FUTX_E_ARG, "weights %s: buffers must be 16-byte aligned", name);
  return FUTX_OK;
}

}  // namespace futx

using namespace futx;

extern "C" {

const char* futx_last_error(void) { return g_err; }

futx_status futx_packed_sizes(const futx_dims* dims, futx_proj proj, size_t* packed_bytes,
                              size_t* scale_bytes) {
  clear_error();
  futx_status st = check_dims(dims);
  if (st || (st = check_proj(proj))) return st;
  if (!packed_bytes || !scale_bytes) return fail(FUTX_E_ARG, "null output pointer");
  ProjShape s = proj_shape(*dims, proj);
  *packed_bytes = (size_t)s.n * s.k / 2;
  *scale_bytes = 2 * scale_count(s.n, s.k / kTileK, dims->w_group);
  return FUTX_OK;
}

futx_status futx_pack_weights_host(const futx_dims* dims, futx_proj proj, const float* w_host,
                                   const float* gain_host, void* packed_host, void* scales_host) {
  clear_error();
  return pack_host(dims, proj, w_host, gain_host, packed_host, scales_host);
}

futx_status futx_pack_weights(const futx_dims* dims, futx_proj proj, const float* w_host,
                              const float* gain_host, void* packed_dev, void* scales_dev,
                              void* stream) {
  clear_error();
  size_t pb, sb;
  futx_status st = futx_packed_sizes(dims, proj, &pb, &sb);
  if (st) return st;
  if (!packed_dev || !scales_dev) return fail(FUTX_E_ARG, "pack: null device pointer");
  std::vector<uint8_t> hp(pb);
  std::vector<uint8_t> hs(sb);
  st = pack_host(dims, proj, w_host, gain_host, hp.data(), hs.data());
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  FUTX_HIP(hipMemcpyAsync(packed_dev, hp.data(), pb, hipMemcpyHostToDevice, s), "pack: copy");
  FUTX_HIP(hipMemcpyAsync(scales_dev, hs.data(), sb, hipMemcpyHostToDevice, s), "pack: copy");
  FUTX_HIP(hipStreamSynchronize(s), "pack: sync");
  return FUTX_OK;
}

futx_status futx_pack_codes_host(const futx_dims* dims, futx_proj proj, const uint8_t* codes_host,
                                 const uint16_t* scales_host, void* packed_host, void* packed_scales_host) {
  clear_error();
  return pack_codes_host(dims, proj, codes_host, scales_host, packed_host, packed_scales_host);
}

futx_status futx_pack_codes(const futx_dims* dims, futx_proj proj, const uint8_t* codes_host,
                            const uint16_t* scales_host, void* packed_dev, void* scales_dev, void* stream) {
  clear_error();
  size_t pb, sb;
  futx_status st = futx_packed_sizes(dims, proj, &pb, &sb);
  if (st) return st;
  if (!packed_dev || !scales_dev) return fail(FUTX_E_ARG, "pack_codes: null device pointer");
  std::vector<uint8_t> hp(pb);
  std::vector<uint8_t> hs(sb);
  st = pack_codes_host(dims, proj, codes_host, scales_host, hp.data(), hs.data());
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  FUTX_HIP(hipMemcpyAsync(packed_dev, hp.data(), pb, hipMemcpyHostToDevice, s), "pack_codes: copy");
  FUTX_HIP(hipMemcpyAsync(scales_dev, hs.data(), sb, hipMemcpyHostToDevice, s), "pack_codes: copy");
  FUTX_HIP(hipStreamSynchronize(s), "pack_codes: sync");
  return FUTX_OK;
}

futx_status futx_unpack_weights(const futx_dims* dims, futx_proj proj, const void* packed_dev,
                                const void* scales_dev, uint8_t* canon_bytes_host,
                                uint16_t* canon_scales_host, void* stream) {
  clear_error();
  size_t pb, sb;
  futx_status st = futx_packed_sizes(dims, proj, &pb, &sb);
  if (st) return st;
  if (!packed_dev || !scales_dev || !canon_bytes_host || !canon_scales_host)
    return fail(FUTX_E_ARG, "unpack: null pointer");
  std::vector<uint8_t> hp(pb), hs(sb);
  hipStream_t s = (hipStream_t)stream;
  FUTX_HIP(hipMemcpyAsync(hp.data(), packed_dev, pb, hipMemcpyDeviceToHost, s), "unpack: copy");
  FUTX_HIP(hipMemcpyAsync(hs.data(), scales_dev, sb, hipMemcpyDeviceToHost, s), "unpack: copy");
  FUTX_HIP(hipStreamSynchronize(s), "unpack: sync");
  return unpack_host(dims, proj, hp.data(), hs.data(), canon_bytes_host, canon_scales_host);
}

futx_status futx_kv_cache_sizes(const futx_dims* dims, int32_t num_pages, size_t* code_bytes,
                                size_t* scale_bytes) {
  clear_error();
  futx_status st = check_dims(dims);
  if (st) return st;
  if (num_pages <= 0 || !code_bytes || !scale_bytes) return fail(FUTX_E_ARG, "kv sizes: bad args");
  *code_bytes = (size_t)num_pages * dims->n_kv_heads * kPageSize * dims->head_dim / 2;
  *scale_bytes = (size_t)num_pages * dims->n_kv_heads * kPageSize * 2;
  return FUTX_OK;
}

futx_status futx_kv_append(const futx_dims* dims, int32_t n_tokens, const float* k, const float* v,
                           const int32_t* positions, const int32_t* slots, uint32_t flags,
                           const futx_kv_cache* cache, void* stream) {
  clear_error();
  futx_status st = check_dims(dims);
  if (st || (st = check_cache(cache))) return st;
  if (n_tokens < 0) return fail(FUTX_E_ARG, "kv_append: negative token count");
  if (n_tokens == 0) return FUTX_OK;
  if (!k || !v || !slots || ((flags & FUTX_KV_ROPE) && !positions))
    return fail(FUTX_E_ARG, "kv_append: null pointer");
  if (flags & ~(FUTX_KV_ROPE | FUTX_KV_HADAMARD)) return fail(FUTX_E_ARG, "kv_append: unknown flags");
  hipError_t e = launch_kv_append(k, v, positions, slots, n_tokens, flags, dims->head_dim,
                                  dims->had_block, dims->rope_theta,
                                  kv_ptrs(cache, dims->n_kv_heads), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv_append: launch");
  return FUTX_OK;
}

futx_status futx_decode_workspace_size(const futx_dims* dims, int32_t max_batch,
                                       int32_t max_context, size_t* bytes) {
  clear_error();
  futx_status st = check_dims(dims);
  if (st) return st;
  if (max_batch < 1 || max_batch > kMaxBatch || max_context < 1 || !bytes)
    return fail(FUTX_E_ARG, "workspace size: batch must be 1..32 and context >= 1");
  // the split plan rounds per batch size, so the largest carve over every
  // batch up to max_batch covers any call with batch <= max_batch
  size_t m = 0;
  for (int b = 1; b <= max_batch; ++b) {
    const size_t v = carve(*dims, b, max_context, nullptr).bytes;
    if (v > m) m = v;
  }
  *bytes = m;
  return FUTX_OK;
}

}  // extern "C"

namespace futx {
size_t decode_workspace_bytes(const futx_dims& d, int batch, int max_context) {
  return carve(d, batch, max_context, nullptr).bytes;
}
}  // namespace futx

// stage < 0: every stage in order; otherwise that stage only
futx_status futx::decode_block_impl(const futx_dims* dims, const futx_block_weights* w, int32_t batch,
                                     float* x, const int32_t* cached_lens, const int32_t* block_table,
                                     int32_t max_pages_per_seq, int32_t max_context,
                                     const futx_kv_cache* cache, void* workspace, size_t workspace_bytes,
                                     void* stream, int stage) {
  clear_error();
  futx_status st = check_dims(dims);
  if (st || (st = check_cache(cache))) return st;
  if (!w) return fail(FUTX_E_ARG, "decode_block: weights is NULL");
  if ((st = check_qweight(&w->qkv, "qkv")) || (st = check_qweight(&w->o, "o")) ||
      (st = check_qweight(&w->gateup, "gateup")) || (st = check_qweight(&w->down, "down")))
    return st;
  if (batch < 1 || batch > kMaxBatch) return fail(FUTX_E_ARG, "decode_block: batch must be 1..32");
  if (!x || !cached_lens || !block_table || !workspace)
    return fail(FUTX_E_ARG, "decode_block: null pointer");
  if (max_pages_per_seq < 1 || max_context < 1 ||
      (long)max_pages_per_seq * kPageSize < (long)max_context)
    return fail(FUTX_E_ARG, "decode_block: max_context exceeds the block table");
  const futx_dims& d = *dims;
  Ws ws = carve(d, batch, max_context, (char*)workspace);
  if (ws.bytes > workspace_bytes)
    return fail(FUTX_E_WORKSPACE, "decode_block: workspace %zu < %zu bytes", workspace_bytes, ws.bytes);
  hipStream_t s = (hipStream_t)stream;
  const int B = batch, H = d.hidden, D = d.head_dim, nq = d.n_heads, G = d.w_group;
  const int nqkv = (d.n_heads + 2 * d.n_kv_heads) * D, I = d.intermediate;
  const KVPtrs kv = kv_ptrs(cache, d.n_kv_heads);
  const size_t term = (size_t)kMaxBatch * kmax(d);
  hipError_t e;
  auto run = [stage](int k) { return stage < 0 || stage == k; };
#define STEP(call)                                             \
  do {                                                         \
    if ((e = (call)) != hipSuccess) return hip_fail(e, #call); \
  } while (0)
  // One INT4 projection with its fused epilogue.  When the activation range
  // does not fit in LDS for this batch, K is split (partial sums) and the
  // epilogue runs as separate kernels.
  auto gemm = [&](const futx_qweight& q, int N, int K, const void* act, int nterms, bool f32, int epi,
                  const float* resid, float* out, uint16_t* out_bf16) -> hipError_t {
    GemmArgs a{};
    a.w = (const uint4*)q.packed;
    a.sc = (const uint16_t*)q.scales;
    a.act = act;
    a.term_stride = term;
    a.N = N;
    a.K = K;
    a.B = B;
    a.eps = d.rms_eps;
    a.resid = resid;
    a.out = out;
    a.out_bf16 = out_bf16;
    a.inter = I;
    if (gemm_fits(N, K, G, B, nterms, epi)) {
      apply_plan(a, plan_gemm(N, K, G, B, nterms, epi));
      return launch_int4_gemm(a, G, nterms, f32, epi, s);
    }
    const GemmPlan2 p = plan_gemm(N, K, G, B, nterms, kEpiPartial);
    apply_plan(a, p);
    a.out = ws.part;
    hipError_t e2 = launch_int4_gemm(a, G, nterms, f32, kEpiPartial, s);
    if (e2 != hipSuccess) return e2;
    switch (epi) {
      case kEpiRms:
        if ((e2 = launch_prep_act((const float*)act, B, K, d.rms_eps, nullptr, ws.invr, s)) != hipSuccess) return e2;
        return launch_reduce(ws.part, p.splits, B, N, ws.invr, nullptr, out, 0, s);
      case kEpiResid:
        return launch_reduce(ws.part, p.splits, B, N, nullptr, resid, out, 0, s);
      case kEpiSwiglu:
        if ((e2 = launch_prep_act((const float*)act, B, K, d.rms_eps, nullptr, ws.invr2, s)) != hipSuccess) return e2;
        return launch_swiglu(ws.part, p.splits, B, I, ws.invr2, out_bf16, s);
    }
    return hipErrorInvalidValue;
  };
  // RMSNorm-1 + QKV (the gain is folded into the weights; 1/r in the epilogue)
  if (run(FUTX_STAGE_QKV)) STEP(gemm(w->qkv, nqkv, H, x, 1, true, kEpiRms, nullptr, ws.qkv, nullptr));
  // RoPE, rotation and INT4 append of the new token, rotated queries,
  // attention over positions 0..cached_lens[b] in splits (one kernel), the
  // merge of the splits and the inverse rotation (a second kernel unless the
  // plan has one workgroup per sequence) -> the O projection operand
  // (FUTX_O_TERMS bf16 terms)
  if (run(FUTX_STAGE_ATTENTION)) {
    AttnArgs aa{};
    aa.qkv = ws.qkv;
    aa.cached_lens = cached_lens;
    aa.block_table = block_table;
    aa.mpps = max_pages_per_seq;
    aa.nq = nq;
    aa.hb = d.had_block;
    aa.tmax = max_context;
    aa.theta = d.rope_theta;
    aa.kv = kv;
    aa.wpart = ws.apart;
    aa.out_bf16 = ws.act;
    aa.term_stride = term;
    STEP(launch_attn_decode(aa, B, D, attn_plan(B, d.n_kv_heads, max_context), s));
  }
  // O projection + residual: h = x + O(o)
  if (run(FUTX_STAGE_O)) STEP(gemm(w->o, H, nq * D, ws.act, FUTX_O_TERMS, false, kEpiResid, x, ws.h, nullptr));
  // RMSNorm-2 + gate/up + SwiGLU -> bf16 activation
  if (run(FUTX_STAGE_GATEUP)) STEP(gemm(w->gateup, 2 * I, H, ws.h, 1, true, kEpiSwiglu, nullptr, nullptr, ws.act));
  // down projection + residual: x = h + down(act)
  if (run(FUTX_STAGE_DOWN)) STEP(gemm(w->down, H, I, ws.act, 1, false, kEpiResid, ws.h, x, nullptr));
#undef STEP
  return FUTX_OK;
}

extern "C" {

futx_status futx_decode_block(const futx_dims* dims, const futx_block_weights* w, int32_t batch,
                              float* x, const int32_t* cached_lens, const int32_t* block_table,
                              int32_t max_pages_per_seq, int32_t max_context,
                              const futx_kv_cache* cache, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return decode_block_impl(dims, w, batch, x, cached_lens, block_table, max_pages_per_seq, max_context,
                           cache, workspace, workspace_bytes, stream, -1);
}

futx_status futx_decode_block_stage(const futx_dims* dims, const futx_block_weights* w, int32_t batch,
                                    float* x, const int32_t* cached_lens, const int32_t* block_table,
                                    int32_t max_pages_per_seq, int32_t max_context,
                                    const futx_kv_cache* cache, void* workspace, size_t workspace_bytes,
                                    int32_t stage, void* stream) {
  if (stage < 0 || stage >= FUTX_STAGE_COUNT) {
    clear_error();
    return fail(FUTX_E_ARG, "decode_block_stage: stage %d out of range", (int)stage);
  }
  return decode_block_impl(dims, w, batch, x, cached_lens, block_table, max_pages_per_seq, max_context,
                           cache, workspace, workspace_bytes, stream, stage);
}

futx_status futx_int4_linear(const futx_dims* dims, futx_proj proj, const futx_qweight* w,
                             int32_t batch, const uint16_t* act, float* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  clear_error();
  futx_status st = check_dims(dims);
  if (st || (st = check_proj(proj)) || (st = check_qweight(w, "linear"))) return st;
  if (batch < 1 || batch > kMaxBatch || !act || !out || !workspace)
    return fail(FUTX_E_ARG, "int4_linear: bad args");
  Ws ws = carve(*dims, batch, 1, (char*)workspace);
  if (ws.bytes > workspace_bytes)
    return fail(FUTX_E_WORKSPACE, "int4_linear: workspace %zu < %zu bytes", workspace_bytes, ws.bytes);
  ProjShape ps = proj_shape(*dims, proj);
  hipStream_t s = (hipStream_t)stream;
  GemmArgs a{};
  a.w = (const uint4*)w->packed;
  a.sc = (const uint16_t*)w->scales;
  a.act = act;
  a.N = ps.n;
  a.K = ps.k;
  a.B = batch;
  a.out = ws.part;
  const GemmPlan2 p = plan_gemm(ps.n, ps.k, dims->w_group, batch, 1, kEpiPartial);
  apply_plan(a, p);
  hipError_t e = launch_int4_gemm(a, dims->w_group, 1, false, kEpiPartial, s);
  if (e != hipSuccess) return hip_fail(e, "int4_linear: gemm");
  e = launch_reduce(ws.part, p.splits, batch, ps.n, nullptr, nullptr, out,
                    proj == FUTX_PROJ_GATEUP ? dims->intermediate : 0, s);
  if (e != hipSuccess) return hip_fail(e, "int4_linear: reduce");
  return FUTX_OK;
}

futx_status futx_decode_attention(const futx_dims* dims, int32_t batch, const float* qkv,
                                  const int32_t* cached_lens, const int32_t* block_table,
                                  int32_t max_pages_per_seq, int32_t max_context,
                                  const futx_kv_cache* cache, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  clear_error();
  futx_status st = check_dims(dims);
  if (st || (st = check_cache(cache))) return st;
  if (batch < 1 || batch > kMaxBatch || !qkv || !cached_lens || !block_table || !out || !workspace)
    return fail(FUTX_E_ARG, "decode_attention: bad args");
  if (max_pages_per_seq < 1 || max_context < 1 ||
      (long)max_pages_per_seq * kPageSize < (long)max_context)
    return fail(FUTX_E_ARG, "decode_attention: max_context exceeds the block table");
  const futx_dims& d = *dims;
  Ws ws = carve(d, batch, max_context, (char*)workspace);
  if (ws.bytes > workspace_bytes)
    return fail(FUTX_E_WORKSPACE, "decode_attention: workspace %zu < %zu bytes", workspace_bytes, ws.bytes);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  AttnArgs aa{};
  aa.qkv = qkv;
  aa.cached_lens = cached_lens;
  aa.block_table = block_table;
  aa.mpps = max_pages_per_seq;
  aa.nq = d.n_heads;
  aa.hb = d.had_block;
  aa.tmax = max_context;
  aa.theta = d.rope_theta;
  aa.kv = kv_ptrs(cache, d.n_kv_heads);
  aa.wpart = ws.apart;
  aa.out_f32 = out;
  if ((e = launch_attn_decode(aa, batch, d.head_dim, attn_plan(batch, d.n_kv_heads, max_context), s)) !=
      hipSuccess)
    return hip_fail(e, "decode_attention");
  return FUTX_OK;
}

futx_status futx_embed(int32_t hidden, int32_t vocab, const uint16_t* table_bf16,
                       const int32_t* tokens, int32_t batch, float* x, void* stream) {
  clear_error();
  if (hidden <= 0 || vocab <= 0) return fail(FUTX_E_ARG, "embed: hidden and vocab must be positive");
  if (batch < 1 || batch > kMaxBatch) return fail(FUTX_E_ARG, "embed: batch must be 1..32");
  if (!table_bf16 || !tokens || !x) return fail(FUTX_E_ARG, "embed: null pointer");
  hipError_t e = launch_embed(table_bf16, tokens, vocab, hidden, batch, x, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "embed");
  return FUTX_OK;
}

futx_status futx_lm_head_workspace_size(const futx_dims* dims, int32_t vocab, int32_t max_batch, size_t* bytes) {
  clear_error();
  futx_status st = check_dims(dims);
  if (st) return st;
  if (vocab <= 0 || max_batch < 1 || max_batch > kMaxBatch || !bytes)
    return fail(FUTX_E_ARG, "lm_head_workspace_size: bad arguments");
  if (!head_shape_ok(dims->hidden)) return fail(FUTX_E_UNSUPPORTED, "lm_head: hidden must be a multiple of 256");
  *bytes = head_ws(dims->hidden, vocab, max_batch, nullptr).bytes;
  return FUTX_OK;
}

futx_status futx_lm_head(const futx_dims* dims, int32_t vocab, const uint16_t* w_bf16,
                         int32_t batch, const float* x, float* logits, int32_t* top1,
                         void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  futx_status st = check_dims(dims);
  if (st) return st;
  if (vocab <= 0) return fail(FUTX_E_ARG, "lm_head: vocab must be positive");
  if (batch < 1 || batch > kMaxBatch) return fail(FUTX_E_ARG, "lm_head: batch must be 1..32");
  if (!w_bf16 || !x || !logits || !top1 || !workspace) return fail(FUTX_E_ARG, "lm_head: null pointer");
  if (((uintptr_t)w_bf16 | (uintptr_t)workspace) & 15) return fail(FUTX_E_ARG, "lm_head: pointers must be 16-byte aligned");
  if (!head_shape_ok(dims->hidden)) return fail(FUTX_E_UNSUPPORTED, "lm_head: hidden must be a multiple of 256");
  const HeadWs ws = head_ws(dims->hidden, vocab, batch, (char*)workspace);
  if (ws.bytes > workspace_bytes)
    return fail(FUTX_E_WORKSPACE, "lm_head: workspace %zu < %zu bytes", workspace_bytes, ws.bytes);
  hipError_t e = launch_lm_head(w_bf16, x, batch, dims->hidden, vocab, dims->rms_eps, ws, logits, top1,
                                (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "lm_head");
  return FUTX_OK;
}

futx_status futx_fold_head(int32_t vocab, int32_t hidden, const uint16_t* w_bf16_host,
                           const float* gain_host, uint16_t* out_bf16_host) {
  clear_error();
  return fold_head_host(vocab, hidden, w_bf16_host, gain_host, out_bf16_host);
}

}  // extern "C"
