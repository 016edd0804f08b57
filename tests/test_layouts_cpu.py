"""The test-side cache decoder: the whole-cache decoder equals the per-page
decoders, and nibble extraction equals a bit-by-bit reading of the encoding
(element e in bits 3..6 of the word rotated right by 4 (e // 2) + 16 (e % 2))."""

import numpy as np
import pytest

from tests import layouts as L


@pytest.mark.parametrize("d", [64, 128])
def test_decode_cache_matches_page_decoders(d):
    r = np.random.default_rng(d)
    P, nkv = 5, 3
    kc = r.integers(0, 256, P * nkv * 64 * d // 2, dtype=np.uint8)
    vc = r.integers(0, 256, P * nkv * 64 * d // 2, dtype=np.uint8)
    ks = r.integers(0, 65535, P * nkv * 64, dtype=np.uint16)
    vs = r.integers(0, 65535, P * nkv * 64, dtype=np.uint16)
    K, KS, V, VS = L.decode_cache(kc, vc, ks, vs, P, nkv, d)
    kc2, vc2 = kc.reshape(P, nkv, -1), vc.reshape(P, nkv, -1)
    for p in range(P):
        for h in range(nkv):
            np.testing.assert_array_equal(K[p, h], L.decode_k_page(kc2[p, h], d))
            np.testing.assert_array_equal(V[p, h], L.decode_v_page(vc2[p, h], d))
    np.testing.assert_array_equal(KS.view(np.uint16).ravel(), ks)
    np.testing.assert_array_equal(VS.view(np.uint16).ravel(), vs)


def test_nibbles_bitwise():
    w = np.random.default_rng(1).integers(0, 2 ** 32, 2000, dtype=np.uint64)
    n = L._nibbles(w.astype(np.uint32))
    for e in range(8):
        rr = 4 * (e // 2) + 16 * (e % 2)
        bits = [(int(x) >> ((rr + 3 + i) % 32)) & 1 for x in w[:50] for i in range(4)]
        want = np.array([sum(bits[4 * j + i] << i for i in range(4)) - 8 for j in range(50)])
        np.testing.assert_array_equal(n[:50, e], want)
