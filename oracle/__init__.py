"""CPU oracle for the INT4 decode block -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, fp64 numpy statement of what the INT4 decode
step of a Llama-style Transformer block computes.  It exists to check the HIP
implementation; it is never part of the product path.  Only the test suite,
the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library and
imports nothing from the ``int4_weight_kv_amd`` package.

Sources (web pages about FuTransformer, "FP8 prefill and INT4 decode for
Llama-style inference on Hopper"):

* [ABS]  the paper's English abstract (airebao.com item page): decode uses
  INT4 projection weights and an INT4 KV-cache copy; a block-diagonal
  Hadamard transform reduces cache quantization error; the kernels are
  checked against a quantized reference computation.
* [INT4] kongchang.com/en article, section "INT4 Decode: letting
  dequantization feed directly into MMA operands" (and its Chinese twin on
  kongchang.com): keys and weights dequantize straight into matrix-core
  operands; the rotation is applied before caching and undone after use.
* [FP8]  same article, section "FP8 Prefill: fusing GEMM and epilogue all the
  way": the fixed RMSNorm gain is folded into the following weights.
* [ACC]  same article, section "Accuracy cost: perplexity from 6.24 to
  7.23": weights are quantized by round-to-nearest (RTN).

The pages print no formula, table or worked example.  Every format detail the
pages leave open (group size, scale type, nibble order, Hadamard block size,
RoPE convention, precision of intermediates) is a documented reading; each
module states the readings it uses.

Floating point: everything is fp64 except (i) the two quantizers, which follow
an exact fp32 recipe so that codes can be compared bit for bit, and (ii) the
bf16 rounding points R1, R3, R4 (R5 for the LM head), where the GPU
materializes bf16 matrix-core operands; the oracle rounds there too, once,
from fp64.  (The attention output is not rounded: the GPU passes it to the O
projection as two bf16 terms, relative error at most 2^-18.)

Parity status per function is listed in each module's docstring.  Functions
with no independent pin say "parity unpinned".
"""

from .numerics import bf16_round, fp16_round_from_fp32
from .quant import (
    quantize_weight_rtn,
    quantize_kv_token,
    pack_nibbles,
    unpack_nibbles,
    dequant_weight,
    fold_gain,
)
from .hadamard import sylvester, hadamard_normalized, block_diag_rotate
from .rope import rope_rotate_half, rope_inv_freq
from .attention import (
    decode_attention,
    attention_bruteforce_loops,
    attention_chunked,
    softmax_merge,
)
from .block import (
    BlockDims,
    QuantBlockWeights,
    LogicalKVCache,
    quantize_block_weights,
    rmsnorm_stats,
    silu,
    history_fill,
    decode_block,
    decode_block_unquantized,
    rotate_kv,
    lm_head,
    fold_head,
    decode_step,
)

__all__ = [name for name in dir() if not name.startswith("_")]
