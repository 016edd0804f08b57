/*
 * futx -- INT4 decode step of a Llama-style Transformer block on AMD Instinct
 * MI355X (gfx950).  C ABI of libfutx.so.
 *
 * Sources.  The method is described by web pages about FuTransformer
 * ("FP8 prefill and INT4 decode for Llama-style inference on Hopper"):
 *   [ABS]  the paper's English abstract (airebao.com item page);
 *   [INT4] kongchang.com/en article, section "INT4 Decode: letting
 *          dequantization feed directly into MMA operands";
 *   [FP8]  same article, section "FP8 Prefill: fusing GEMM and epilogue all
 *          the way";
 *   [ACC]  same article, section "Accuracy cost: perplexity from 6.24 to 7.23".
 * The decode block uses INT4 projection weights and an INT4 KV-cache copy
 * [ABS]; weights and keys are stored so that dequantized values feed the
 * matrix cores directly, without an intermediate tile in memory [ABS, INT4];
 * a block-diagonal Hadamard rotation reduces cache quantization error from
 * outlier channels [ABS]; the RMSNorm gain is folded into the weights that
 * follow the norm [ABS, FP8]; weights are rounded to nearest [ACC].
 *
 * Conventions (all entry points):
 *  - Every buffer is owned by the caller.  The library allocates no device
 *    memory and keeps no pointer after the call returns.
 *  - "dev" pointers are device memory of the current HIP device; "host"
 *    pointers are host memory.  `stream` is a hipStream_t (NULL = the null
 *    stream).  Device work is enqueued asynchronously on `stream` unless the
 *    entry point says otherwise.
 *  - Arguments are validated on the host before anything is enqueued; on a
 *    negative status nothing has been enqueued and futx_last_error() returns
 *    a message (thread-local).  Device-side metadata (lengths, block tables,
 *    slots, token ids) is trusted: out-of-range values are undefined
 *    behaviour.
 *  - No C++ exception crosses the ABI.  Calls are reentrant; calls on one
 *    stream run in order.
 *
 * Number formats:
 *  - bf16 / fp16 buffers are passed as uint16_t bit patterns.
 *  - INT4 codes are symmetric, in [-8, 7]; a group of `w_group` input
 *    channels of one weight row shares one fp16 scale = fp16(max|w| / 7)
 *    (fp32 arithmetic, round to nearest even) and codes are
 *    clamp(rint(w / scale), -8, 7) with the stored scale as divisor.  The KV
 *    cache uses the same recipe with one scale per (token, KV head) over all
 *    head_dim channels, saturated at 65504.
 */
#ifndef FUTX_H
#define FUTX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t futx_status;
#define FUTX_OK 0
#define FUTX_E_ARG (-1)         /* null pointer, negative or inconsistent size */
#define FUTX_E_UNSUPPORTED (-2) /* a shape or option the kernels do not support */
#define FUTX_E_WORKSPACE (-3)   /* workspace smaller than required */
#define FUTX_E_RANGE (-4)       /* a weight group scale overflows fp16 */
#define FUTX_E_HIP (-5)         /* a HIP runtime call failed */

/* Shape of one decoder block.  Supported: head_dim in {64, 128}; w_group in
 * {64, 128}; had_block in {32, 64} dividing head_dim; page_size 64;
 * hidden, n_heads*head_dim and intermediate multiples of 128 and of
 * 2*w_group (an even number of scale groups per weight row); head_dim a multiple of w_group; n_heads a multiple of n_kv_heads
 * with n_heads / n_kv_heads <= 16. */
typedef struct futx_dims {
  int32_t hidden;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t intermediate;
  int32_t w_group;   /* weight quantization group along the input dimension */
  int32_t had_block; /* block size of the block-diagonal Hadamard rotation */
  int32_t page_size; /* KV-cache tokens per page */
  float rms_eps;     /* RMSNorm epsilon */
  float rope_theta;  /* RoPE base */
} futx_dims;

/* The four projections of a block.  Logical weight matrices are row-major
 * [N][K] fp32 (row n = output feature n, column k = input feature k):
 *   QKV    N = (n_heads + 2 n_kv_heads) head_dim, K = hidden; rows are the
 *          query heads, then the key heads, then the value heads, each head
 *          head_dim consecutive rows.
 *   O      N = hidden, K = n_heads head_dim.
 *   GATEUP N = 2 intermediate, K = hidden; rows 0..I-1 are the gate
 *          projection, rows I..2I-1 the up projection.
 *   DOWN   N = hidden, K = intermediate. */
typedef enum futx_proj {
  FUTX_PROJ_QKV = 0,
  FUTX_PROJ_O = 1,
  FUTX_PROJ_GATEUP = 2,
  FUTX_PROJ_DOWN = 3
} futx_proj;

/* Packed INT4 weights of one projection in device memory, in the order
 * futx_pack_weights writes (opaque to callers; 256-byte aligned). */
typedef struct futx_qweight {
  const void* packed; /* futx_packed_sizes(...).packed_bytes bytes */
  const void* scales; /* futx_packed_sizes(...).scale_bytes bytes (fp16) */
} futx_qweight;

typedef struct futx_block_weights {
  futx_qweight qkv, o, gateup, down;
} futx_block_weights;

/* Paged INT4 KV cache of one layer (device memory, caller-owned).  Token t
 * of a sequence lives in physical page block_table[t / page_size] at offset
 * t % page_size; a "slot" is page * page_size + offset.  The code buffers
 * hold the rotated keys and values in the order the attention kernel reads
 * them (opaque; futx_kv_cache_sizes gives the sizes).  Scales are fp16
 * [num_pages][n_kv_heads][page_size]. */
typedef struct futx_kv_cache {
  void* k_codes;
  void* v_codes;
  void* k_scales;
  void* v_scales;
  int32_t num_pages;
} futx_kv_cache;

/* Flags of futx_kv_append. */
#define FUTX_KV_ROPE 1u     /* apply RoPE to keys at `positions` */
#define FUTX_KV_HADAMARD 2u /* rotate keys and values by the block Hadamard */

/* Last error message of this thread ("" if none). */
const char* futx_last_error(void);

/* ------------------------------------------------------------------ weights */

/* Device bytes of a packed projection.  Source: INT4 projection weights
 * with per-group scales [ABS, ACC]. */
futx_status futx_packed_sizes(const futx_dims* dims, futx_proj proj, size_t* packed_bytes,
                              size_t* scale_bytes);

/* Offline weight packing.  Folds the RMSNorm gain into the weight columns
 * (w'[n][k] = w[n][k] * gain[k], one fp32 multiply) when `gain_host` is not
 * NULL [ABS, FP8], quantizes w' by the INT4 recipe above [ACC] and reorders
 * nibbles and scales into the matrix-core operand order of the kernels
 * [ABS, INT4].  w_host: fp32 [N][K] row-major (host).  gain_host: fp32 [K]
 * or NULL (QKV takes the attention-norm gain, GATEUP the MLP-norm gain).
 * Writes packed_dev / scales_dev (sizes from futx_packed_sizes) and returns
 * after the copies have completed.  FUTX_E_RANGE if a scale overflows fp16. */
futx_status futx_pack_weights(const futx_dims* dims, futx_proj proj, const float* w_host,
                              const float* gain_host, void* packed_dev, void* scales_dev,
                              void* stream);

/* Same as futx_pack_weights but writes the device-order bytes to host
 * buffers (no HIP call). */
futx_status futx_pack_weights_host(const futx_dims* dims, futx_proj proj, const float* w_host,
                                   const float* gain_host, void* packed_host, void* scales_host);

/* Ingestion of codes quantized elsewhere in the same format (the pages name
 * GPTQ weights "in the same format" as the alternative to round-to-nearest
 * [ACC]): canonical bytes [N][K/2] (byte i of a row = code 2i in the low
 * nibble, code 2i+1 in the high nibble, two's complement, every code in
 * [-8, 7] accepted) and fp16 scales [N][K/w_group] in logical row order
 * (host), reordered into the device order of futx_pack_weights.  No folding
 * or quantization happens: a gain must already be in the codes and scales.
 * FUTX_E_RANGE if a scale is not a finite fp16 value.  Returns after the
 * copies have completed. */
futx_status futx_pack_codes(const futx_dims* dims, futx_proj proj, const uint8_t* codes_host,
                            const uint16_t* scales_host, void* packed_dev, void* scales_dev,
                            void* stream);

/* Same as futx_pack_codes but writes the device-order bytes to host buffers
 * (no HIP call). */
futx_status futx_pack_codes_host(const futx_dims* dims, futx_proj proj, const uint8_t* codes_host,
                                 const uint16_t* scales_host, void* packed_host,
                                 void* packed_scales_host);

/* Inverse of the device order (for tests; the device order is the operand
 * order in which the dequantized values feed the matrix cores [INT4]): reads
 * packed_dev / scales_dev and writes canonical bytes [N][K/2] (byte i of a row = code 2i in the low
 * nibble, code 2i+1 in the high nibble, two's complement) and fp16 scales
 * [N][K/w_group] in logical row order (host).  Blocks until done. */
futx_status futx_unpack_weights(const futx_dims* dims, futx_proj proj, const void* packed_dev,
                                const void* scales_dev, uint8_t* canon_bytes_host,
                                uint16_t* canon_scales_host, void* stream);

/* ----------------------------------------------------------------- KV cache */

/* Bytes of each code buffer (k_codes and v_codes have the same size) and of
 * each scale buffer for `num_pages` pages of the INT4 cache copy [INT4]: per
 * page, KV head and token, head_dim / 2 code bytes for keys and as many for
 * values, and one fp16 scale each. */
futx_status futx_kv_cache_sizes(const futx_dims* dims, int32_t num_pages, size_t* code_bytes,
                                size_t* scale_bytes);

/* Write n_tokens tokens into the INT4 cache [ABS]: for each token and KV
 * head, keys get RoPE at positions[i] (FUTX_KV_ROPE), keys and values get
 * the block-Hadamard rotation (FUTX_KV_HADAMARD) [ABS, INT4], then each is
 * quantized per (token, KV head) and stored at slots[i].  flags = 0 stores
 * the inputs as given (quantizer only).  k, v: fp32 [n_tokens][n_kv_heads]
 * [head_dim] (dev, pre-RoPE keys); positions, slots: int32 [n_tokens] (dev).
 * Slots must be distinct within one call. */
futx_status futx_kv_append(const futx_dims* dims, int32_t n_tokens, const float* k, const float* v,
                           const int32_t* positions, const int32_t* slots, uint32_t flags,
                           const futx_kv_cache* cache, void* stream);

/* ------------------------------------------------------------- decode block */

/* Workspace bytes of futx_decode_block for up to `max_batch` sequences
 * (1..32) of up to `max_context` cached tokens: the decode block of [ABS] at
 * the batches the pages measure (1..32), its intermediate activations and
 * attention partials (caller-owned; the library allocates nothing). */
futx_status futx_decode_workspace_size(const futx_dims* dims, int32_t max_batch,
                                       int32_t max_context, size_t* bytes);

/* One decode step of one block for `batch` sequences (1..32) [ABS]:
 *   x <- x + O(attn(rope/rotate(QKV(rmsnorm1(x)))))           (residual 1)
 *   x <- x + DOWN(silu(GATE(rmsnorm2(x))) * UP(rmsnorm2(x)))   (residual 2)
 * with INT4 weights dequantized into bf16 matrix-core operands and fp32
 * accumulation [ABS, INT4].  RMSNorm gains are already folded into the QKV
 * and GATEUP weights.  The new token's key and value are rotated, quantized
 * and written to the cache at position cached_lens[b] (slot from the block
 * table) before attention reads positions 0..cached_lens[b] [ABS].
 *   x           fp32 [batch][hidden] (dev), in/out residual stream.
 *   cached_lens int32 [batch] (dev): tokens already cached = the new token's
 *               position.  Not modified; the caller advances it.
 *   block_table int32 [batch][max_pages_per_seq] (dev).
 *   workspace   >= futx_decode_workspace_size(dims, batch, max context) bytes
 *               (dev), contents need not be initialized.
 *   max_context upper bound on cached_lens[b] + 1 over the batch (sizes the
 *               split-sequence attention); must be <= the workspace's.  A
 *               sequence outside it (or with cached_lens[b] < 0) is not
 *               written to the cache and its row of x becomes NaN (the
 *               kernels stay in bounds). */
futx_status futx_decode_block(const futx_dims* dims, const futx_block_weights* w, int32_t batch,
                              float* x, const int32_t* cached_lens, const int32_t* block_table,
                              int32_t max_pages_per_seq, int32_t max_context,
                              const futx_kv_cache* cache, void* workspace, size_t workspace_bytes,
                              void* stream);

/* futx_decode_block without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels, launch order
 * and results as futx_decode_block, with the workspace taken from a static
 * device buffer of 72 MiB that the library holds on each GPU it runs on
 * until the process ends (enough for the 70B shape at batch 32).  It calls
 * no allocating routine.  FUTX_E_WORKSPACE if batch and max_context need
 * more scratch than that (use futx_decode_block).  Every call on a GPU
 * shares that GPU's buffer: calls that overlap on one GPU (several streams
 * or threads) race; calls on one stream run in order. */
futx_status futx_decode_block_noalloc(const futx_dims* dims, const futx_block_weights* w, int32_t batch,
                                      float* x, const int32_t* cached_lens, const int32_t* block_table,
                                      int32_t max_pages_per_seq, int32_t max_context,
                                      const futx_kv_cache* cache, void* stream);

/* Stages of futx_decode_block, in launch order (one kernel each; the
 * attention stage adds a merge kernel when the plan splits a sequence over
 * more than one workgroup). */
#define FUTX_STAGE_QKV 0        /* RMSNorm-1 scale + QKV projection */
#define FUTX_STAGE_ATTENTION 1  /* RoPE, block rotation and INT4 append of the new token, rotated
                                   queries, split-sequence attention, merge of the splits and the
                                   inverse rotation */
#define FUTX_STAGE_O 2          /* O projection + residual 1 */
#define FUTX_STAGE_GATEUP 3     /* RMSNorm-2 scale + gate/up projection + SwiGLU */
#define FUTX_STAGE_DOWN 4       /* down projection + residual 2 */
#define FUTX_STAGE_COUNT 5

/* Runs one stage of futx_decode_block with the same kernels, launch
 * configuration and workspace, for per-kernel timing (same arguments, plus
 * `stage` in [0, FUTX_STAGE_COUNT)).  A stage reads what the stages before it
 * left in the workspace and cache, so call futx_decode_block once first for
 * meaningful values; every stage is safe to repeat (the append rewrites the
 * same slot, the projections recompute their outputs).  FUTX_E_ARG for a
 * stage out of range; otherwise as futx_decode_block. */
futx_status futx_decode_block_stage(const futx_dims* dims, const futx_block_weights* w, int32_t batch,
                                    float* x, const int32_t* cached_lens, const int32_t* block_table,
                                    int32_t max_pages_per_seq, int32_t max_context,
                                    const futx_kv_cache* cache, void* workspace, size_t workspace_bytes,
                                    int32_t stage, void* stream);

/* ------------------------------------------------------ component entry points
 * Single steps of the block, for tests and profiling. */

/* out[b][n] = sum_k act[b][k] * (code[n][k] * scale[n][k / w_group]) for one
 * packed projection: act bf16 [batch][K] (dev), out fp32 [batch][N] (dev,
 * logical row order).  batch 1..32.  Workspace from futx_decode_workspace_size. */
futx_status futx_int4_linear(const futx_dims* dims, futx_proj proj, const futx_qweight* w,
                             int32_t batch, const uint16_t* act, float* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* The attention stage of futx_decode_block alone, with the same kernel and
 * launch configuration, writing fp32 instead of the O-projection operand
 * [ABS, INT4]: for each sequence b and KV head, the new token's key gets
 * RoPE at position cached_lens[b], its key and value the block-Hadamard
 * rotation; both are quantized per token and written to the cache at slot
 * cached_lens[b]; then query head i attends over positions
 * 0..cached_lens[b] of KV head i / (n_heads / n_kv_heads) with rotated
 * queries, softmax(q k / sqrt(head_dim)) v, and the output is rotated back.
 *   qkv     fp32 [batch][(n_heads + 2 n_kv_heads) head_dim] (dev): the QKV
 *           projection, rows q | k | v head-major, before RoPE.
 *   out     fp32 [batch][n_heads][head_dim] (dev).
 *   other arguments as futx_decode_block.
 * A sequence with cached_lens[b] < 0 or cached_lens[b] + 1 > max_context
 * gets NaN outputs and no cache write (the kernels stay in bounds). */
futx_status futx_decode_attention(const futx_dims* dims, int32_t batch, const float* qkv,
                                  const int32_t* cached_lens, const int32_t* block_table,
                                  int32_t max_pages_per_seq, int32_t max_context,
                                  const futx_kv_cache* cache, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* --------------------------------------------------------- full decode step */

/* Token embedding of the full decode step whose time the pages report per
 * token [ABS]: x[b][:] = fp32(table[tokens[b]][:]) for a bf16 embedding table
 * [vocab][hidden] (dev); tokens int32 [batch] (dev, trusted; out-of-range ids are clamped to
 * [0, vocab)); x fp32 [batch][hidden] (dev).  batch 1..32. */
futx_status futx_embed(int32_t hidden, int32_t vocab, const uint16_t* table_bf16,
                       const int32_t* tokens, int32_t batch, float* x, void* stream);

/* LM head with the final RMSNorm [FP8 folding, ABS]: logits[b][v] =
 * (sum_k bf16(x[b][k]) w[v][k]) / r_b with r_b = sqrt(mean_k x[b][k]^2 + eps),
 * fp32 accumulation, and top1[b] = the lowest index of the largest logit.
 *   w_bf16  [vocab][hidden] bf16 (dev, 16-byte aligned), final norm gain
 *           already folded in (futx_fold_head).
 *   x       fp32 [batch][hidden] (dev); logits fp32 [batch][vocab] (dev);
 *           top1 int32 [batch] (dev).  batch 1..32.
 *   workspace >= futx_lm_head_workspace_size(dims, vocab, batch) bytes (dev,
 *           16-byte aligned), contents need not be initialized.
 * FUTX_E_UNSUPPORTED unless dims->hidden is a multiple of 256. */
futx_status futx_lm_head(const futx_dims* dims, int32_t vocab, const uint16_t* w_bf16,
                         int32_t batch, const float* x, float* logits, int32_t* top1,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of futx_lm_head for up to `max_batch` rows (1..32).
 * FUTX_E_UNSUPPORTED unless dims->hidden is a multiple of 256. */
futx_status futx_lm_head_workspace_size(const futx_dims* dims, int32_t vocab, int32_t max_batch,
                                        size_t* bytes);

/* Host-side fold of the final norm gain into the bf16 LM head:
 * out[v][k] = bf16(fp32(w[v][k]) * gain[k]) (round to nearest even). */
futx_status futx_fold_head(int32_t vocab, int32_t hidden, const uint16_t* w_bf16_host,
                           const float* gain_host, uint16_t* out_bf16_host);

/* ---------------------------------------------------------- FP8 comparison
 * The pages set the INT4 decode path against the authors' FP8 path (the
 * INT4 decode block is 31-51% faster [ABS]).  These entries give the same
 * projection with e4m3 weights and activations on the fp8 matrix cores.
 * Format (a reading; the pages give none): OCP e4m3 "fn" bytes (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits; largest finite 448), one fp32
 * scale per group of 128 inputs for weight rows and for activation rows,
 * s = fp32(max|x| / 448), codes e4m3(fp32(x / s)) rounded to nearest even,
 * saturated at 448.  Rows stay in logical order (gate then up for GATEUP);
 * the weight bytes are in the fp8 matrix-core operand order (opaque). */

/* Device bytes of an FP8-packed projection: packed = N K, scales = 4 N K / 128. */
futx_status futx_fp8_packed_sizes(const futx_dims* dims, futx_proj proj, size_t* packed_bytes,
                                  size_t* scale_bytes);

/* Offline FP8 packing: folds `gain_host` (or NULL) into the columns like
 * futx_pack_weights, quantizes by the recipe above and writes the device
 * order.  w_host fp32 [N][K] (host).  Returns after the copies completed. */
futx_status futx_pack_fp8_weights(const futx_dims* dims, futx_proj proj, const float* w_host,
                                  const float* gain_host, void* packed_dev, void* scales_dev, void* stream);

/* Same, writing host buffers (no HIP call). */
futx_status futx_pack_fp8_weights_host(const futx_dims* dims, futx_proj proj, const float* w_host,
                                       const float* gain_host, void* packed_host, void* scales_host);

/* Workspace bytes of futx_fp8_linear for up to `max_batch` rows (1..32). */
futx_status futx_fp8_linear_workspace_size(const futx_dims* dims, futx_proj proj, int32_t max_batch,
                                           size_t* bytes);

/* Activation quantization by the recipe above: act bf16 [rows][k] (dev) ->
 * codes e4m3 bytes [rows][k] and scales fp32 [rows][k / 128] (dev, caller
 * owned).  k a positive multiple of 128, rows 1..65535; asynchronous on
 * `stream`.  The division x / s is IEEE fp32, so the codes equal a host
 * computation of the same recipe bit for bit. */
futx_status futx_fp8_quantize_act(int32_t k, int32_t rows, const uint16_t* act, uint8_t* codes, float* scales,
                                  void* stream);

/* out[b][n] = sum_g s_w[n][g] s_a[b][g] sum_{k in g} w[n][k] a[b][k]: the
 * activation rows act (bf16 [batch][K], dev) are quantized on the device by
 * futx_fp8_quantize_act into the workspace, then multiplied on the fp8 matrix
 * cores; out fp32 [batch][N] (dev).  w: an FP8-packed projection.
 * Accuracy: the gfx950 fp8 matrix instruction sums each run of 8 products
 * after truncating them toward zero to 13 bits below the run's largest
 * operand exponent sum, so the group sums are not exact products summed in
 * fp32 (the per-output bound is stated with the GPU parity test). */
futx_status futx_fp8_linear(const futx_dims* dims, futx_proj proj, const futx_qweight* w, int32_t batch,
                            const uint16_t* act, float* out, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------- measurement */

/* Plain streaming read of `bytes` (a positive multiple of 16) of device
 * memory at `buf` (16-byte aligned) by `workgroups` workgroups of 256
 * threads, each reading one contiguous chunk with 128-bit loads: the
 * achievable HBM read bandwidth that the decode kernels are compared with
 * (decode is bound by weight and KV-cache reads: kongchang.com/en article,
 * section "Why do Prefill and Decode need different quantization
 * strategies?").  sink: uint32 [workgroups] (dev), written only in the rare
 * case that a workgroup's XOR of its data equals a fixed value (it keeps the
 * loads from being optimized away). */
futx_status futx_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FUTX_H */
