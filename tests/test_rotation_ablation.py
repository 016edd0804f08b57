"""Rotation ablation on the oracle: the block-diagonal Hadamard rotation
lowers the INT4 cache error caused by outlier key channels.

The pages state the effect without numbers: rotating K/V by a block-diagonal
Hadamard transform before per-token INT4 quantization spreads outlier
channels and reduces the cache's quantization error (FuTransformer abstract,
airebao.com item page; kongchang.com/en, section "INT4 Decode: letting
dequantization feed directly into MMA operands").  These tests check the
direction on the outlier-key workload (4 of 128 channels per KV head x16
before RoPE), and that without outliers the rotation changes nothing material.
The same comparison on the device cache is in test_gpu_parity.py.
"""

import numpy as np

import oracle
from int4_weight_kv_amd import workload as W


def _cache_roundtrip(x, hb, rotate):
    """x [T][nkv][d] fp64 -> dequantized cache content in x's own basis."""
    y = oracle.block_diag_rotate(x, hb) if rotate else x
    codes, scales = oracle.quantize_kv_token(y.astype(np.float32))
    deq = codes.astype(np.float64) * scales.astype(np.float64)[..., None]
    return oracle.block_diag_rotate(deq, hb) if rotate else deq


def _rel(a, ref):
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


def _keys_values(wl, n=512):
    d = wl.dims
    k, v = W.history(wl, 0, 0, n)
    pos = np.arange(n)[:, None]
    k_rope = oracle.rope_rotate_half(k.astype(np.float64), pos, d.rope_theta)
    return k_rope, v.astype(np.float64)


def ablation(wl, n=512, seed=5):
    """Relative errors (Frobenius) of the dequantized cache and of the
    attention output against the unquantized fp64 values, without and with
    the rotation."""
    d = wl.dims
    k, v = _keys_values(wl, n)
    q = np.random.default_rng(seed).standard_normal((d.n_heads, d.head_dim))
    ref = oracle.decode_attention(q, k, v, 1)  # hb = 1: no rotation anywhere
    out = {}
    for rot in (False, True):
        kh = _cache_roundtrip(k, d.had_block, rot)
        vh = _cache_roundtrip(v, d.had_block, rot)
        tag = "rot" if rot else "plain"
        out[f"k_{tag}"] = _rel(kh, k)
        out[f"v_{tag}"] = _rel(vh, v)
        out[f"attn_{tag}"] = _rel(oracle.decode_attention(q, kh, vh, 1), ref)
    return out


def test_rotation_cuts_outlier_key_error():
    e = ablation(W.llama8b_ragged(1))
    # outlier keys: the rotation spreads the x16 channels over each 64-block
    assert e["k_rot"] < 0.5 * e["k_plain"], e
    assert e["attn_rot"] < e["attn_plain"], e
    # values carry no outliers: the rotation neither helps nor hurts much
    assert abs(e["v_rot"] - e["v_plain"]) < 0.05 * e["v_plain"], e


def test_rotation_neutral_without_outliers():
    e = ablation(W.llama8b())
    assert abs(e["k_rot"] - e["k_plain"]) < 0.05 * e["k_plain"], e
    assert abs(e["v_rot"] - e["v_plain"]) < 0.05 * e["v_plain"], e


def test_rotation_is_exactly_undone_without_quantization():
    """Rotating and rotating back is the identity (the normalized Sylvester
    matrix is symmetric and orthogonal), so any error above comes from the
    quantizer alone."""
    wl = W.llama8b_ragged(1)
    k, _ = _keys_values(wl, 64)
    hb = wl.dims.had_block
    np.testing.assert_allclose(oracle.block_diag_rotate(oracle.block_diag_rotate(k, hb), hb), k, atol=1e-12)


if __name__ == "__main__":
    for wl in (W.llama8b_ragged(1), W.llama8b()):
        print(wl.name, {k: round(v, 4) for k, v in ablation(wl).items()})
