"""The FP8 host packer (futx_pack_fp8_weights_host) writes exactly the
oracle's e4m3 codes and fp32 group scales (oracle/fp8.py), with the gain
folded in, in the documented device order (decoded by tests/layouts.py)."""

import numpy as np
import pytest

import oracle
from oracle import fp8
from int4_weight_kv_amd import workload as W
from tests import layouts


@pytest.fixture(scope="module")
def fx():
    from int4_weight_kv_amd import futx

    return futx


@pytest.mark.parametrize("proj", ["qkv", "o", "gateup", "down"])
def test_fp8_pack_bit_exact_tiny(fx, proj):
    wl = W.tiny()
    d = wl.dims
    w = W.block_weights(wl, 0)
    m, g = {"qkv": (w["wqkv"], w["gain_attn"]), "o": (w["wo"], None),
            "gateup": (np.concatenate([w["wgate"], w["wup"]]), w["gain_ffn"]), "down": (w["wdown"], None)}[proj]
    m = m.copy()
    m[0, :128] = 0.0  # a zero group
    m[1, 5] = -0.0
    pb, sb = fx.futx_fp8_packed_sizes(d, proj)
    n, k = m.shape
    assert pb == n * k and sb == n * (k // 128) * 4
    packed, scales = np.zeros(pb, np.uint8), np.zeros(sb, np.uint8)
    fx.futx_pack_fp8_weights_host(d, proj, m, g, packed, scales)
    codes, s = layouts.decode_fp8_weights(packed, scales, n, k)
    folded = m if g is None else oracle.fold_gain(m, g)
    want_c, want_s = fp8.quantize_groups(folded)
    np.testing.assert_array_equal(s.view(np.uint32), want_s.view(np.uint32))
    np.testing.assert_array_equal(codes, want_c)


def test_fp8_pack_8b_down_bit_exact(fx):
    d = W.LLAMA8B
    r = np.random.default_rng(9)
    m = (r.standard_normal((d.hidden, d.intermediate)) * 0.02).astype(np.float32)
    m[7, 300:700] *= 50.0  # groups with larger range
    pb, sb = fx.futx_fp8_packed_sizes(d, "down")
    packed, scales = np.zeros(pb, np.uint8), np.zeros(sb, np.uint8)
    fx.futx_pack_fp8_weights_host(d, "down", m, None, packed, scales)
    codes, s = layouts.decode_fp8_weights(packed, scales, d.hidden, d.intermediate)
    want_c, want_s = fp8.quantize_groups(m)
    np.testing.assert_array_equal(s.view(np.uint32), want_s.view(np.uint32))
    np.testing.assert_array_equal(codes, want_c)
