"""Pins of the FP8 (e4m3) oracle (oracle/fp8.py): the decode of every byte
against torch's float8_e4m3fn (a library routine), the encoder against
torch's cast and hand-derived codes (tests/golden/fp8_cases.txt), the
round-trip bound of the group quantizer, and the projection against a
brute-force sum; planted mistakes are caught."""

import os

import numpy as np
import pytest

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_cases.txt")
torch = pytest.importorskip("torch")


def _cases():
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            v, code, _ = [p.strip() for p in line.split("|")]
            yield float(v), int(code, 16)


def test_decode_all_bytes_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.e4m3_decode(b)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])


def test_encode_hand_cases():
    for v, code in _cases():
        assert int(fp8.e4m3_encode(np.float32(v))) == code, (v, hex(code))


def test_encode_matches_torch_within_range():
    r = np.random.default_rng(0)
    v = np.concatenate([
        (r.standard_normal(20000) * 60).astype(np.float32),
        r.uniform(-464, 464, 20000).astype(np.float32),
        (r.standard_normal(5000) * 0.01).astype(np.float32),  # subnormals and small normals
        np.ldexp(r.integers(-15, 16, 4000) + 0.5, r.integers(-12, 6, 4000)).astype(np.float32),  # ties
        np.array([0.0, -0.0, 448.0, -448.0, 464.0], np.float32),
    ])
    v = v[np.abs(v) <= 464]
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(fp8.e4m3_encode(v), want)


def test_group_quantizer_roundtrip_and_zero():
    r = np.random.default_rng(1)
    x = (r.standard_normal((16, 512)) * np.exp(r.standard_normal((16, 1)))).astype(np.float32)
    x[3, 128:256] = 0.0
    codes, s = fp8.quantize_groups(x)
    assert s.dtype == np.float32 and s.shape == (16, 4)
    assert s[3, 1] == 0 and np.all(codes[3, 128:256] == 0)
    deq = fp8.dequant_groups(codes, s)
    v = fp8.e4m3_decode(codes)
    # half a step of the code's binade: 2^(E - 4) for |v| in [2^E, 2^(E+1)), 2^-10 below 2^-6
    _, ex = np.frexp(np.abs(v))
    half = np.where(np.abs(v) < 2.0 ** -6, 2.0 ** -10, np.ldexp(1.0, ex - 5))
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(x - deq) <= half * sf * (1 + 1e-6) + 1e-30)
    # the largest element of every nonzero group reaches the top of the range
    amax = np.abs(v).reshape(16, 4, 128).max(axis=2)
    assert np.all(amax[s > 0] >= 447.0)


def test_linear_matches_bruteforce():
    r = np.random.default_rng(2)
    B, N, K = 3, 5, 256
    a = r.standard_normal((B, K)).astype(np.float32)
    w = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    wc, ws = fp8.quantize_groups(w)
    ac, as_ = fp8.quantize_groups(a)
    got = fp8.fp8_linear(a, wc, ws)
    for b in range(B):
        for n in range(N):
            tot = 0.0
            for g in range(K // 128):
                part = 0.0
                for k in range(g * 128, (g + 1) * 128):
                    part += float(fp8.e4m3_decode(wc[n, k])) * float(fp8.e4m3_decode(ac[b, k]))
                tot += float(ws[n, g]) * float(as_[b, g]) * part
            assert abs(got[b, n] - tot) <= 1e-12 * max(1.0, abs(tot))


def test_planted_rounding_mistake_is_caught(monkeypatch):
    real_rint = np.rint

    class _NP:
        def __getattr__(self, name):
            return getattr(np, name)

        @staticmethod
        def rint(x):  # ties away from zero instead of to even
            return np.floor(np.asarray(x) + 0.5)

    monkeypatch.setattr(fp8, "np", _NP())
    with pytest.raises(AssertionError):
        test_encode_hand_cases()
    assert real_rint is np.rint


def test_planted_bias_mistake_is_caught(monkeypatch):
    real = fp8.e4m3_decode
    monkeypatch.setattr(fp8, "e4m3_decode", lambda c: real(c) * 2.0)  # exponent bias 6 instead of 7
    with pytest.raises(AssertionError):
        test_decode_all_bytes_matches_torch()
