"""Composed-oracle checks: the decode block on the tiny shape against an
unquantized fp64 block (sanity: quantization-noise-sized differences only),
history fill consistency, and planted mistakes that the pins must catch."""

import numpy as np
import pytest

import oracle
from int4_weight_kv_amd import workload as W


def _tiny_setup(batch, lengths, outliers=False, seed=0):
    wl = W.Workload(f"oracle-test-b{batch}", W.TINY, batch, "fixed:0", outliers=outliers)
    dims = wl.dims
    w = W.block_weights(wl, 0, seed)
    qw = oracle.quantize_block_weights(w, dims)
    x = W.hidden_state(wl, seed)
    caches, kh, vh = [], [], []
    for b, L in enumerate(lengths):
        k, v = W.history(wl, 0, b, L, seed)
        c = oracle.LogicalKVCache.empty(L + 1, dims.n_kv_heads, dims.head_dim)
        oracle.history_fill(c, k, v, np.arange(L), dims)
        caches.append(c)
        kh.append(k)
        vh.append(v)
    return wl, dims, w, qw, x, caches, kh, vh


@pytest.mark.parametrize("batch,lengths", [(1, [128]), (3, [0, 5, 70])])
def test_block_close_to_unquantized(batch, lengths):
    wl, dims, w, qw, x, caches, kh, vh = _tiny_setup(batch, lengths)
    y = oracle.decode_block(x, qw, caches, np.array(lengths), dims)
    y_ref = oracle.decode_block_unquantized(x, w, kh, vh, np.array(lengths), dims)
    delta = y_ref - x
    rel = np.linalg.norm(y - y_ref) / np.linalg.norm(delta)
    assert 1e-3 < rel < 0.3, rel  # INT4 noise (~11% per projection): visible but bounded
    # unrotated unquantized block is the same function (rotation is exact in fp64)
    y_nr = oracle.decode_block_unquantized(x, w, kh, vh, np.array(lengths), dims, rotate=False)
    np.testing.assert_allclose(y_nr, y_ref, rtol=0, atol=1e-10)


def test_block_appends_new_token():
    wl, dims, w, qw, x, caches, _, _ = _tiny_setup(2, [3, 9])
    diag = {}
    oracle.decode_block(x, qw, caches, np.array([3, 9]), dims, diag=diag)
    nq, nkv, d = dims.n_heads, dims.n_kv_heads, dims.head_dim
    for b, L in enumerate([3, 9]):
        k = diag["qkv"][b, nq * d:(nq + nkv) * d].reshape(nkv, d)
        v = diag["qkv"][b, (nq + nkv) * d:].reshape(nkv, d)
        kr, vr = oracle.rotate_kv(k, v, L, dims)
        kc, ks = oracle.quantize_kv_token(kr.astype(np.float32))
        np.testing.assert_array_equal(caches[b].k_codes[L], kc)
        np.testing.assert_array_equal(caches[b].k_scales[L], ks)
        vc, vs = oracle.quantize_kv_token(vr.astype(np.float32))
        np.testing.assert_array_equal(caches[b].v_codes[L], vc)


def test_outlier_rotation_reduces_cache_error():
    """Direction of the pages' claim: rotating before INT4 lowers the cache
    error on keys with outlier channels."""
    wl = W.Workload("oracle-outlier", W.LLAMA8B, 1, "fixed:0", outliers=True)
    k, _ = W.history(wl, 0, 0, 256)
    dims = wl.dims
    pos = np.arange(256)[:, None]
    k_rope = oracle.rope_rotate_half(k.astype(np.float64), pos, dims.rope_theta)
    k_rot = oracle.block_diag_rotate(k_rope, dims.had_block)
    q1, s1 = oracle.quantize_kv_token(k_rope.astype(np.float32))
    q2, s2 = oracle.quantize_kv_token(k_rot.astype(np.float32))
    e_plain = np.linalg.norm(q1 * s1[..., None].astype(np.float64) - k_rope)
    e_rot = np.linalg.norm(oracle.block_diag_rotate(q2 * s2[..., None].astype(np.float64), dims.had_block) - k_rope)
    assert e_rot < 0.6 * e_plain


# ------------------------------------------------------------ planted mistakes


def test_planted_rope_sign_error_is_caught(monkeypatch):
    from oracle import rope as orope

    def bad(x, pos, theta):
        x = np.asarray(x, np.float64)
        d = x.shape[-1]
        ang = np.asarray(pos, np.float64)[..., None] * orope.rope_inv_freq(d, theta)
        c, s = np.cos(ang), np.sin(ang)
        a, b = x[..., : d // 2], x[..., d // 2:]
        return np.concatenate([a * c + b * s, b * c + a * s], axis=-1)  # wrong sign

    monkeypatch.setattr(oracle, "rope_rotate_half", bad)
    from tests import test_oracle_pins as pins

    with pytest.raises(AssertionError):
        pins.test_rope_hand_cases()
    with pytest.raises(AssertionError):
        pins.test_rope_invariants()


def test_planted_merge_error_is_caught(monkeypatch):
    from oracle import attention as oatt

    def bad_merge(parts):
        m = max(p[0] for p in parts)
        return sum(p[2] for p in parts) / sum(p[1] for p in parts)  # forgets the rescale

    monkeypatch.setattr(oatt, "softmax_merge", bad_merge)
    from tests import test_oracle_pins as pins

    with pytest.raises(AssertionError):
        pins.test_attention_chunked_equals_full()


def test_planted_transposed_hadamard_block_is_caught(monkeypatch):
    from oracle import hadamard as oh

    def bad_rotate(x, hb):  # strided blocks instead of contiguous ones
        x = np.asarray(x, np.float64)
        d = x.shape[-1]
        h = oh.hadamard_normalized(hb)
        xb = x.reshape(x.shape[:-1] + (hb, d // hb))
        return np.swapaxes(np.swapaxes(xb, -1, -2) @ h.T, -1, -2).reshape(x.shape)

    monkeypatch.setattr(oracle, "block_diag_rotate", bad_rotate)
    from tests import test_oracle_pins as pins

    with pytest.raises(AssertionError):
        pins.test_block_rotation_preserves_dot_products()


def test_planted_quant_divisor_error_is_caught(monkeypatch):
    from oracle import quant as oq

    def bad(g32, saturate):  # divides by the unrounded fp32 scale
        g32 = np.asarray(g32, np.float32)
        a = np.max(np.abs(g32), axis=-1)
        s32 = (a / np.float32(7.0)).astype(np.float32)
        s16 = s32.astype(np.float16)
        sf = s32[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            r = (g32 / sf).astype(np.float32)
        q = np.where(sf == 0, 0, np.clip(np.rint(r), -8, 7))
        return q.astype(np.int8), s16

    monkeypatch.setattr(oq, "_quantize_groups_fp32", bad)
    from tests import test_oracle_pins as pins

    with pytest.raises(AssertionError):
        pins.test_quant_hand_cases("weight")
