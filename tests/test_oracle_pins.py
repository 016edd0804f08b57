"""Pins of the CPU oracle against facts fixed outside the oracle itself:
hand-derived cases (tests/golden), closed forms, invariants, library routines
(scipy's Hadamard, torch's bf16 cast) and brute force on tiny inputs."""

import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oatt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [p.strip() for p in line.split("|")]


# ---------------------------------------------------------------- rounding


def test_bf16_round_matches_torch_cast():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(1)
    vals = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(5000) * 1e30).astype(np.float32),
        (r.standard_normal(5000) * 1e-38).astype(np.float32),  # subnormal range
        np.array([1.0, -1.0, 0.0, 65504.0, 3.0e38], np.float32),
    ])
    # exact ties: low 16 bits = 0x8000, with even and odd kept LSB
    bits = r.integers(0x3F000000, 0x40800000, size=4000, dtype=np.uint32)
    ties = ((bits & 0xFFFF0000) | 0x8000).astype(np.uint32).view(np.float32)
    vals = np.concatenate([vals, ties])
    want = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(vals.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_round_single_rounding_from_fp64():
    # 1 + 2**-8 + 2**-30 lies just above the tie between 1 and 1 + 2**-7:
    # one rounding from fp64 goes up; a detour through fp32 would hit the tie.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.bf16_round(np.array([x]))[0] == 1.0 + 2.0 ** -7


# ---------------------------------------------------------------- quantizers


@pytest.mark.parametrize("kind", ["weight", "kv"])
def test_quant_hand_cases(kind):
    for inp, scale, codes in _rows("quant_cases.txt"):
        w = np.array([float(v) for v in inp.split()], np.float32)
        if kind == "weight":
            q, s = oracle.quantize_weight_rtn(w[None, :], 4)
            q, s = q[0], s[0, 0]
        else:
            q, s = oracle.quantize_kv_token(w[None, :])
            q, s = q[0], s[0]
        assert float(s) == float(scale), (inp, float(s))
        np.testing.assert_array_equal(q, [int(c) for c in codes.split()])


@pytest.mark.parametrize("group", [64, 128])
def test_weight_roundtrip_bound(group):
    r = np.random.default_rng(2)
    w = (r.standard_normal((64, 512)) * 0.02).astype(np.float32)
    w[3, :group] = 0.0  # one zero group
    q, s = oracle.quantize_weight_rtn(w, group)
    assert q.min() >= -7 and q.max() <= 7  # -8 is unreachable with max|w|/7
    sf = np.repeat(s.astype(np.float64), group, axis=1)
    err = np.abs(w.astype(np.float64) - q * sf)
    assert np.all(err <= sf / 2 + 1e-30)
    assert np.all(q[3, :group] == 0) and s[3, 0] == 0
    # every nonzero group uses its full code range at the max element
    nz = s.astype(np.float64) > 0
    amax = np.abs(q).reshape(64, -1, group).max(axis=2)
    assert np.all(amax[nz] == 7)


def test_kv_roundtrip_bound_and_saturation():
    r = np.random.default_rng(3)
    x = r.standard_normal((100, 8, 128)).astype(np.float32)
    q, s = oracle.quantize_kv_token(x)
    sf = s.astype(np.float64)[..., None]
    assert np.all(np.abs(x - q * sf) <= sf / 2 + 1e-30)
    big = np.full((1, 4), 1e6, np.float32)
    q, s = oracle.quantize_kv_token(big)
    assert float(s[0]) == 65504.0 and np.all(q == 7)
    with pytest.raises(OverflowError):
        oracle.quantize_weight_rtn(big, 4)


def test_pack_hand_cases_and_exhaustive():
    for codes, hexb in _rows("pack_cases.txt"):
        c = np.array([int(v) for v in codes.split()], np.int8)
        want = np.array([int(h, 16) for h in hexb.split()], np.uint8)
        np.testing.assert_array_equal(oracle.pack_nibbles(c), want)
        np.testing.assert_array_equal(oracle.unpack_nibbles(want), c)
    allb = np.arange(256, dtype=np.uint8)
    np.testing.assert_array_equal(oracle.pack_nibbles(oracle.unpack_nibbles(allb)), allb)


def test_fold_identity():
    r = np.random.default_rng(4)
    x = r.standard_normal((3, 64))
    w = r.standard_normal((32, 64))
    gam = r.uniform(0.5, 1.5, 64)
    rr = oracle.rmsnorm_stats(x, 1e-5)
    lhs = ((x / rr[:, None]) * gam) @ w.T
    rhs = (x / rr[:, None]) @ (w * gam[None, :]).T
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)
    # the fp32 fold is one fp32 multiply per element
    w32, g32 = w.astype(np.float32), gam.astype(np.float32)
    np.testing.assert_array_equal(oracle.fold_gain(w32, g32), np.float32(w32 * g32))


# ---------------------------------------------------------------- Hadamard


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64, 128])
def test_hadamard_orthogonal_and_library(n):
    scipy_linalg = pytest.importorskip("scipy.linalg")
    h = oracle.sylvester(n)
    np.testing.assert_array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))
    np.testing.assert_array_equal(h, scipy_linalg.hadamard(n))
    hn = oracle.hadamard_normalized(n)
    np.testing.assert_allclose(hn, hn.T, atol=0)
    np.testing.assert_allclose(hn @ hn, np.eye(n), atol=1e-14)


def test_hadamard_hand_cases():
    for n, inp, out in _rows("hadamard_cases.txt"):
        n = int(n)
        if inp.startswith("dense="):
            x = np.array([float(v) for v in inp[6:].split(",")])
            want = np.array([float(v) for v in out.split(",")])
        else:
            x = np.zeros(n)
            for kv in inp.split():
                i, v = kv.split("=")
                x[int(i)] = float(v)
            want = np.full(n, float(out))
        np.testing.assert_allclose(oracle.block_diag_rotate(x, n), want, rtol=0, atol=1e-14)


def test_block_rotation_preserves_dot_products():
    r = np.random.default_rng(5)
    q = r.standard_normal((6, 128))
    k = r.standard_normal((9, 128))
    for hb in (32, 64):
        qr, kr = oracle.block_diag_rotate(q, hb), oracle.block_diag_rotate(k, hb)
        np.testing.assert_allclose(qr @ kr.T, q @ k.T, rtol=0, atol=1e-12)
        # blocks are contiguous: rotating only the first block leaves the rest alone
        x = np.zeros(128)
        x[hb:] = r.standard_normal(128 - hb)
        np.testing.assert_allclose(oracle.block_diag_rotate(x, hb)[hb:],
                                   oracle.block_diag_rotate(x[hb:], hb), atol=1e-14)


# ---------------------------------------------------------------- RoPE


def test_rope_hand_cases():
    for theta, pos, inp, out in _rows("rope_cases.txt"):
        x = np.array([float(v) for v in inp.split()])
        want = np.array([float(v) for v in out.split()])
        got = oracle.rope_rotate_half(x, int(pos), float(theta))
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_rope_invariants():
    r = np.random.default_rng(6)
    d = 128
    q, k = r.standard_normal(d), r.standard_normal(d)
    for theta in (10000.0, 500000.0):
        np.testing.assert_allclose(oracle.rope_rotate_half(q, 0, theta), q, atol=0)
        qr = oracle.rope_rotate_half(q, 777, theta)
        np.testing.assert_allclose(qr[:64] ** 2 + qr[64:] ** 2, q[:64] ** 2 + q[64:] ** 2, rtol=1e-12)
        a = oracle.rope_rotate_half(q, 1000, theta) @ oracle.rope_rotate_half(k, 990, theta)
        b = oracle.rope_rotate_half(q, 20, theta) @ oracle.rope_rotate_half(k, 10, theta)
        assert abs(a - b) < 1e-9
    # theta is not hard-coded: different theta gives a different rotation
    assert not np.allclose(oracle.rope_rotate_half(q, 5, 10000.0), oracle.rope_rotate_half(q, 5, 500000.0))


# ---------------------------------------------------------------- attention


def _rand_attn(r, t_len, nq=4, nkv=2, d=64):
    return (r.standard_normal((nq, d)), r.standard_normal((t_len, nkv, d)), r.standard_normal((t_len, nkv, d)))


def test_attention_matches_bruteforce_loops():
    r = np.random.default_rng(7)
    for t_len in (1, 2, 7, 33):
        q, k, v = _rand_attn(r, t_len)
        got = oracle.decode_attention(q, k, v, 32)
        want = oracle.attention_bruteforce_loops(q.tolist(), k.tolist(), v.tolist(), 32)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_attention_chunked_equals_full():
    r = np.random.default_rng(8)
    q, k, v = _rand_attn(r, 300, nq=8, nkv=2, d=128)
    full = oracle.decode_attention(q, k, v, 64)
    for bounds in ([0, 300], [0, 64, 128, 300], [0, 1, 2, 299, 300], [0, 17, 100, 101, 250, 300]):
        np.testing.assert_allclose(oracle.attention_chunked(q, k, v, 64, bounds), full, rtol=0, atol=1e-12)


def test_attention_special_cases():
    r = np.random.default_rng(9)
    q, k, v = _rand_attn(r, 1)
    # a single token (no history): output is the rotated value of that token
    got = oracle.decode_attention(q, k, v, 32)
    for i in range(4):
        np.testing.assert_allclose(got[i], oracle.block_diag_rotate(v[0, i // 2], 32), atol=1e-14)
    # equal scores: the mean of the values
    q = np.zeros((4, 64))
    _, k, v = _rand_attn(r, 10)
    got = oracle.decode_attention(q, k, v, 32)
    np.testing.assert_allclose(got[1], oracle.block_diag_rotate(v[:, 0].mean(axis=0), 32), atol=1e-14)
    np.testing.assert_allclose(got[3], oracle.block_diag_rotate(v[:, 1].mean(axis=0), 32), atol=1e-14)


def test_rotated_attention_equals_unrotated():
    r = np.random.default_rng(10)
    q, k, v = _rand_attn(r, 50, nq=4, nkv=1, d=128)
    hb = 64
    rot = oracle.decode_attention(oracle.block_diag_rotate(q, hb), oracle.block_diag_rotate(k, hb),
                                  oracle.block_diag_rotate(v, hb), hb)
    # unrotated: plain softmax attention (the definition, with loops)
    want = []
    for i in range(4):
        z = k[:, 0] @ q[i] / math.sqrt(128)
        p = np.exp(z - z.max())
        want.append((p / p.sum()) @ v[:, 0])
    np.testing.assert_allclose(rot, np.array(want), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- norm / activation


def test_rmsnorm_and_silu_closed_forms():
    c = 3.0
    x = np.full((1, 256), c)
    rr = oracle.rmsnorm_stats(x, 1e-5)
    np.testing.assert_allclose(x / rr[:, None], c / math.sqrt(c * c + 1e-5), rtol=1e-15)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.silu(np.array([40.0])), [40.0], rtol=1e-15)
    np.testing.assert_allclose(oracle.silu(np.array([-40.0])), [0.0], atol=1e-15)
    np.testing.assert_allclose(oracle.silu(np.array([1.0])), [1.0 / (1.0 + math.exp(-1.0))], rtol=1e-15)
