"""The INT4 decode step of a Llama-style block, end to end (oracle, test infrastructure only).

Step order (pages: [ABS] and [INT4]; readings in the module docstrings of
quant, hadamard, rope and attention):

  O1  fold the RMSNorm gains into the weights that follow the norms
      (QKV <- attention gain, gate/up <- MLP gain) and quantize every
      projection by fp32 RTN (quant.py).
  O4  RMSNorm-1.  Reading: the GPU multiplies the GEMM result by 1/r instead
      of normalizing the operand, so the matrix-core operand is u = bf16(x)
      (rounding point R1) and r = sqrt(mean(x^2) + eps).
  O5  qkv = (W_qkv u) / r; rows are q (n_heads*d), then k, then v, head-major.
  O6  RoPE on q and k at position L_b (the number of cached tokens).
  O7  block Hadamard on q, k and v.
  O8  per (token, KV head) INT4 quantization of k and v (fp32 recipe) and
      append at slot L_b.
  O9  attention over tokens 0..L_b of the cache (the new token read back
      quantized), inverse rotation of the output.
  O10 h = x + W_o o  (o unrounded: the GPU carries the attention output
      into the O projection as a sum of two bf16 terms, relative error at
      most 2^-18, so there is no bf16 rounding point between attention and
      the O projection)
  O11 RMSNorm-2 like O4: u2 = bf16(h), r2 = sqrt(mean(h^2) + eps)     (R3)
  O12 g = (W_gate u2)/r2, v = (W_up u2)/r2, act = bf16(silu(g) v)    (R4)
  O13 y = h + W_down act  -- the block output (fp64 here).
  O14 history fill: earlier tokens' k, v go through O6-O8 at their own
      positions (no projection); it stands in for prefill.
  O15 full step: x0 = Emb[token]; all layers; u = bf16(x) (R5), logits =
      (W_head' u) / r with W_head' = bf16(fp32(W_head * final gain)); top-1 is
      the lowest index of the maximum.

Everything is fp64 except the quantizers (fp32 recipe) and the bf16
rounding points R1 (block input), R3 (MLP input), R4 (SwiGLU output) and R5
(LM-head input), where the GPU materializes bf16 matrix-core operands.

Parity status.  The parts are pinned in tests/test_oracle_pins.py.  The
composition is pinned in tests/test_oracle_closed_forms.py by closed forms:
a constant input row fixes qkv, g and up as bf16(c) times row sums of the
dequantized weights over sqrt(c^2 + eps) (O4/O5, O11/O12); zero O weights
make h = x; eps = 0 makes qkv, g and up invariant under x -> 2^k x; unit
head rows fix the logits and the lowest-index top-1 (O15 tail); zero
projections reduce the step to the head of the embedding row (O15).  The
attention output's path into h (O9 -> O10) and the new token's append are
covered by the attention pins and by the comparison with
``decode_block_unquantized`` (quantization-noise-sized differences only),
which is a sanity check rather than an exact pin.
"""

from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np

from .attention import decode_attention
from .hadamard import block_diag_rotate
from .numerics import bf16_round
from .quant import fold_gain, quantize_kv_token, quantize_weight_rtn
from .rope import rope_rotate_half


@dataclass(frozen=True)
class BlockDims:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    w_group: int
    had_block: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def n_qkv(self):
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def group_q(self):
        return self.n_heads // self.n_kv_heads


@dataclass
class QuantBlockWeights:
    """Codes int8 [N][K] and fp16 scales [N][K/group] of each projection."""

    group: int
    codes: dict
    scales: dict
    _deq: dict = field(default_factory=dict)

    def dense(self, name):
        """Dequantized fp64 matrix q * s (cached)."""
        if name not in self._deq:
            c = self.codes[name]
            n, k = c.shape
            s = self.scales[name].astype(np.float64)
            w = c.reshape(n, k // self.group, self.group).astype(np.float64)
            w *= s[:, :, None]
            self._deq[name] = w.reshape(n, k)
        return self._deq[name]

    def drop_dense(self):
        self._deq.clear()


def quantize_block_weights(w, dims):
    """O1: fold gains, then RTN-quantize.

    ``w`` holds fp32 arrays: wqkv [Nqkv][H], wo [H][nq*d], wgate [I][H],
    wup [I][H], wdown [H][I], gain_attn [H], gain_ffn [H].
    """
    g = dims.w_group
    mats = {
        "qkv": fold_gain(w["wqkv"], w["gain_attn"]),
        "o": np.asarray(w["wo"], np.float32),
        "gate": fold_gain(w["wgate"], w["gain_ffn"]),
        "up": fold_gain(w["wup"], w["gain_ffn"]),
        "down": np.asarray(w["wdown"], np.float32),
    }
    codes, scales = {}, {}
    for name, m in mats.items():
        codes[name], scales[name] = quantize_weight_rtn(m, g)
    return QuantBlockWeights(group=g, codes=codes, scales=scales)


@dataclass
class LogicalKVCache:
    """One sequence's INT4 cache of one layer, in logical token order."""

    k_codes: np.ndarray  # int8 [cap][nkv][d]
    k_scales: np.ndarray  # fp16 [cap][nkv]
    v_codes: np.ndarray
    v_scales: np.ndarray

    @staticmethod
    def empty(cap, nkv, d):
        return LogicalKVCache(
            np.zeros((cap, nkv, d), np.int8),
            np.zeros((cap, nkv), np.float16),
            np.zeros((cap, nkv, d), np.int8),
            np.zeros((cap, nkv), np.float16),
        )

    def write(self, t, kc, ks, vc, vs):
        self.k_codes[t], self.k_scales[t] = kc, ks
        self.v_codes[t], self.v_scales[t] = vc, vs

    def dequant(self, n_tokens):
        k = self.k_codes[:n_tokens].astype(np.float64) * self.k_scales[:n_tokens, :, None].astype(np.float64)
        v = self.v_codes[:n_tokens].astype(np.float64) * self.v_scales[:n_tokens, :, None].astype(np.float64)
        return k, v


def rmsnorm_stats(x, eps):
    """r = sqrt(mean(x^2) + eps) per row, fp64."""
    x = np.asarray(x, np.float64)
    return np.sqrt(np.mean(x * x, axis=-1) + eps)


def silu(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def rotate_kv(k_pre, v, pos, dims):
    """O6-O7 for keys (RoPE then block Hadamard) and values (block Hadamard)."""
    k_rot = block_diag_rotate(rope_rotate_half(k_pre, pos, dims.rope_theta), dims.had_block)
    v_rot = block_diag_rotate(v, dims.had_block)
    return k_rot, v_rot


def history_fill(cache, k_pre, v, positions, dims):
    """O14: write tokens ``positions`` of ``cache`` from pre-RoPE k [T][nkv][d]
    and v [T][nkv][d] (fp32 inputs)."""
    pos = np.asarray(positions)
    k_rot, v_rot = rotate_kv(np.asarray(k_pre, np.float64), np.asarray(v, np.float64), pos[:, None], dims)
    kc, ks = quantize_kv_token(k_rot.astype(np.float32))
    vc, vs = quantize_kv_token(v_rot.astype(np.float32))
    cache.k_codes[pos], cache.k_scales[pos] = kc, ks
    cache.v_codes[pos], cache.v_scales[pos] = vc, vs


def decode_block(x, weights, caches, lens, dims, diag=None, kv_hook=None):
    """O4-O13 for a batch.  ``x`` fp32 [B][H]; ``caches`` one LogicalKVCache per
    sequence (the new token is appended at ``lens[b]``).  Returns y fp64 [B][H].

    ``kv_hook`` (tests only; None leaves the arithmetic as stated): called as
    kv_hook(b, kc, ks, vc, vs, k_rot, v_rot) with the new token's codes and
    scales (O8) and the fp64 rotated k, v they were quantized from; it returns
    the codes and scales to append.  A test uses it to continue with an
    implementation's choice where a value sits on a rounding boundary, after
    checking that the choice is one of the two valid ones."""
    x = np.asarray(x, np.float64)
    bsz = x.shape[0]
    nq, nkv, d = dims.n_heads, dims.n_kv_heads, dims.head_dim
    # O4 / O5
    u = bf16_round(x)
    r = rmsnorm_stats(x, dims.rms_eps)
    qkv = (u @ weights.dense("qkv").T) / r[:, None]
    q = qkv[:, : nq * d].reshape(bsz, nq, d)
    k = qkv[:, nq * d : (nq + nkv) * d].reshape(bsz, nkv, d)
    v = qkv[:, (nq + nkv) * d :].reshape(bsz, nkv, d)
    o = np.empty((bsz, nq, d))
    q_rot_all = np.empty((bsz, nq, d))
    for b in range(bsz):
        pos = int(lens[b])
        # O6 / O7
        q_rot = block_diag_rotate(rope_rotate_half(q[b], pos, dims.rope_theta), dims.had_block)
        k_rot, v_rot = rotate_kv(k[b], v[b], pos, dims)
        # O8
        kc, ks = quantize_kv_token(k_rot.astype(np.float32))
        vc, vs = quantize_kv_token(v_rot.astype(np.float32))
        if kv_hook is not None:
            kc, ks, vc, vs = kv_hook(b, kc, ks, vc, vs, k_rot, v_rot)
        caches[b].write(pos, kc, ks, vc, vs)
        # O9
        k_hat, v_hat = caches[b].dequant(pos + 1)
        o[b] = decode_attention(q_rot, k_hat, v_hat, dims.had_block)
        q_rot_all[b] = q_rot
    # O10 (no rounding point: see the module docstring)
    o_flat = o.reshape(bsz, nq * d)
    h = x + o_flat @ weights.dense("o").T
    # O11 / O12
    u2 = bf16_round(h)
    r2 = rmsnorm_stats(h, dims.rms_eps)
    g = (u2 @ weights.dense("gate").T) / r2[:, None]
    up = (u2 @ weights.dense("up").T) / r2[:, None]
    act = bf16_round(silu(g) * up)
    # O13
    y = h + act @ weights.dense("down").T
    if diag is not None:
        diag.update(u=u, r=r, qkv=qkv, q_rot=q_rot_all, o=o, h=h, u2=u2, r2=r2, g=g, up=up, act=act)
    return y


def decode_block_unquantized(x, w, k_hist, v_hist, lens, dims, rotate=True):
    """Reference without any quantization or bf16 rounding (fp64 weights with
    folded gains, fp64 cache).  Sanity comparison only.

    ``k_hist[b]``/``v_hist[b]`` are pre-RoPE history [L_b][nkv][d]."""
    x = np.asarray(x, np.float64)
    bsz = x.shape[0]
    nq, nkv, d = dims.n_heads, dims.n_kv_heads, dims.head_dim
    wqkv = np.asarray(w["wqkv"], np.float64) * np.asarray(w["gain_attn"], np.float64)[None, :]
    wg = np.asarray(w["wgate"], np.float64) * np.asarray(w["gain_ffn"], np.float64)[None, :]
    wu = np.asarray(w["wup"], np.float64) * np.asarray(w["gain_ffn"], np.float64)[None, :]
    r = rmsnorm_stats(x, dims.rms_eps)
    qkv = (x / r[:, None]) @ wqkv.T
    q = qkv[:, : nq * d].reshape(bsz, nq, d)
    k = qkv[:, nq * d : (nq + nkv) * d].reshape(bsz, nkv, d)
    v = qkv[:, (nq + nkv) * d :].reshape(bsz, nkv, d)
    o = np.empty((bsz, nq, d))
    for b in range(bsz):
        lb = int(lens[b])
        pos_hist = np.arange(lb)[:, None]
        kk = np.concatenate([rope_rotate_half(np.asarray(k_hist[b], np.float64), pos_hist, dims.rope_theta),
                             rope_rotate_half(k[b], lb, dims.rope_theta)[None]], axis=0)
        vv = np.concatenate([np.asarray(v_hist[b], np.float64), v[b][None]], axis=0)
        qq = rope_rotate_half(q[b], lb, dims.rope_theta)
        if rotate:
            kk = block_diag_rotate(kk, dims.had_block)
            vv = block_diag_rotate(vv, dims.had_block)
            qq = block_diag_rotate(qq, dims.had_block)
            o[b] = decode_attention(qq, kk, vv, dims.had_block)
        else:
            # unrotated attention: no output rotation either
            o[b] = block_diag_rotate(decode_attention(qq, kk, vv, dims.had_block), dims.had_block)
    h = x + o.reshape(bsz, nq * d) @ np.asarray(w["wo"], np.float64).T
    r2 = rmsnorm_stats(h, dims.rms_eps)
    u2 = h / r2[:, None]
    act = silu(u2 @ wg.T) * (u2 @ wu.T)
    return h + act @ np.asarray(w["wdown"], np.float64).T


def lm_head(x, w_head_folded, eps):
    """O15 tail: logits = (W' bf16(x)) / r and the lowest-index top-1.

    ``w_head_folded`` holds bf16 values (as float) of fp32(W_head * gain)."""
    x = np.asarray(x, np.float64)
    u = bf16_round(x)
    r = rmsnorm_stats(x, eps)
    logits = (u @ np.asarray(w_head_folded, np.float64).T) / r[:, None]
    return logits, np.argmax(logits, axis=1)


def fold_head(w_head_bf16, gain_final):
    """W_head' = bf16(fp32(W_head * gain[k]))."""
    return bf16_round(fold_gain(np.asarray(w_head_bf16, np.float32), gain_final).astype(np.float64))


def decode_step(tokens, emb_bf16, n_layers, layer_weights: Callable[[int], QuantBlockWeights],
                layer_caches: Callable[[int], List[LogicalKVCache]], lens, dims,
                w_head_folded, progress: Optional[Callable[[int], None]] = None):
    """O15: one full decode step.  ``layer_weights(l)`` / ``layer_caches(l)``
    supply each layer on demand so that only one fp64 layer is alive."""
    x = np.asarray(emb_bf16, np.float64)[np.asarray(tokens)]
    for layer in range(n_layers):
        wq = layer_weights(layer)
        x = decode_block(x.astype(np.float32), wq, layer_caches(layer), lens, dims)
        wq.drop_dense()
        if progress is not None:
            progress(layer)
    return lm_head(x, w_head_folded, dims.rms_eps)
