"""CPU-side checks of the C ABI: the library loads, exports every entry point
of include/futx.h, validates arguments before touching the GPU, and its host
packer writes exactly the codes and scales of the oracle's quantizer in the
documented device order (decoded by tests/layouts.py)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from int4_weight_kv_amd import workload as W
from tests import layouts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "futx.h")


@pytest.fixture(scope="module")
def fx():
    from int4_weight_kv_amd import futx

    return futx


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(futx_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(fx):
    names = _declared()
    assert len(names) >= 15
    lib = ctypes.CDLL(fx.LIBRARY_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    nm = subprocess.run(["nm", "-D", "--defined-only", fx.LIBRARY_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (futx_\w+)", nm))
    assert set(names) <= exported
    assert set(fx.EXPORTED) == set(names)


def test_argument_validation(fx):
    d = fx.make_dims(W.TINY)
    with pytest.raises(fx.FutxError) as e:
        fx.futx_packed_sizes(W.Dims(256, 4, 2, 96, 768, 64, 32), "qkv")
    assert e.value.status == fx.FUTX_E_UNSUPPORTED
    with pytest.raises(fx.FutxError) as e:
        fx.futx_packed_sizes(W.Dims(256, 4, 2, 64, 768, 64, 48), "qkv")
    assert e.value.status == fx.FUTX_E_UNSUPPORTED
    with pytest.raises(fx.FutxError) as e:
        fx.futx_packed_sizes(W.Dims(0, 4, 2, 64, 768, 64, 32), "qkv")
    assert e.value.status == fx.FUTX_E_ARG
    with pytest.raises(fx.FutxError) as e:
        fx.futx_packed_sizes(W.TINY, 7)
    assert e.value.status == fx.FUTX_E_ARG
    with pytest.raises(fx.FutxError) as e:
        fx.futx_decode_workspace_size(W.TINY, 33, 100)
    assert e.value.status == fx.FUTX_E_ARG
    # decode_block rejects a null cache before anything reaches the GPU
    cache = fx.futx_kv_cache(None, None, None, None, 0)
    wts = fx.make_block_weights((None, None), (None, None), (None, None), (None, None))
    with pytest.raises(fx.FutxError) as e:
        fx.futx_decode_block(W.TINY, wts, 1, None, None, None, 1, 1, cache, None, 0, stream=0)
    assert e.value.status == fx.FUTX_E_ARG
    assert "cache" in fx.futx_last_error()


def test_decode_block_stage_range(fx):
    """The stage number is checked before any pointer is used or kernel launched."""
    for bad in (-1, fx.FUTX_STAGE_COUNT):
        with pytest.raises(fx.FutxError) as e:
            fx.futx_decode_block_stage(W.TINY, fx.futx_block_weights(), 1, None, None, None, 1, 1,
                                       fx.futx_kv_cache(), None, 0, bad)
        assert e.value.status == fx.FUTX_E_ARG
        assert "stage" in fx.futx_last_error()


def test_lm_head_workspace_and_validation(fx):
    n = fx.futx_lm_head_workspace_size(W.LLAMA8B, 128256, 16)
    assert n >= 4 * 16 * 128256 * 4  # fp32 partials of four K splits
    assert fx.futx_lm_head_workspace_size(W.LLAMA8B, 128256, 32) >= n
    odd = W.Dims(384, 4, 2, 64, 768, 64, 32)  # hidden not a multiple of 256
    with pytest.raises(fx.FutxError) as e:
        fx.futx_lm_head_workspace_size(odd, 1000, 1)
    assert e.value.status == fx.FUTX_E_UNSUPPORTED
    for bad in (0, 33):
        with pytest.raises(fx.FutxError) as e:
            fx.futx_lm_head(W.LLAMA8B, 1000, None, bad, None, None, None, None, 0)
        assert e.value.status == fx.FUTX_E_ARG
    with pytest.raises(fx.FutxError) as e:
        fx.futx_embed(4096, 1000, None, None, 1, None)
    assert e.value.status == fx.FUTX_E_ARG


def test_noalloc_scratch_bounds(fx):
    """The static buffer of futx_decode_block_noalloc (72 MiB, include/futx.h)
    holds the 70B-shape block at batch 32, and the request the GPU rejection
    test makes (with placeholder buffers) needs more than twice that: that
    test relies on the call being refused before any launch."""
    scratch = 72 << 20
    for mc in (4097, 8193, 131073):
        assert fx.futx_decode_workspace_size(W.llama70b(32).dims, 32, mc) <= scratch
        assert fx.futx_decode_workspace_size(W.LLAMA8B, 32, mc) <= scratch
    big = W.Dims(16384, 64, 8, 128, 229376, 128, 64)
    assert fx.futx_decode_workspace_size(big, 32, 9) > 2 * scratch


def test_sizes(fx):
    pb, sb = fx.futx_packed_sizes(W.LLAMA8B, "gateup")
    assert pb == 2 * 14336 * 4096 // 2 and sb == 2 * 14336 * 32 * 2
    # scales are padded to whole blocks of 8 K blocks: K = 768 has 6
    pb, sb = fx.futx_packed_sizes(W.TINY, "down")
    assert pb == 256 * 768 // 2 and sb == 256 * 8 * 2 * 2
    cb, sb = fx.futx_kv_cache_sizes(W.LLAMA8B, 10)
    assert cb == 10 * 8 * 64 * 64 and sb == 10 * 8 * 64 * 2
    assert fx.futx_decode_workspace_size(W.LLAMA8B, 32, 8192) > fx.futx_decode_workspace_size(W.LLAMA8B, 1, 2048)


def _host_pack(fx, dims, proj, w, gain):
    pb, sb = fx.futx_packed_sizes(dims, proj)
    packed = np.zeros(pb, np.uint8)
    scales = np.zeros(sb // 2, np.uint16)
    fx.futx_pack_weights_host(dims, proj, w, gain, packed, scales)
    return packed, scales


@pytest.mark.parametrize("proj", ["qkv", "o", "gateup", "down"])
def test_host_pack_bit_exact_tiny(fx, proj):
    wl = W.tiny()
    w = W.block_weights(wl, 0)
    d = wl.dims
    mats = {"qkv": (w["wqkv"], w["gain_attn"]), "o": (w["wo"], None),
            "gateup": (np.concatenate([w["wgate"], w["wup"]]), w["gain_ffn"]), "down": (w["wdown"], None)}
    m, g = mats[proj]
    packed, scales = _host_pack(fx, d, proj, m, g)
    n, k = m.shape
    codes = layouts.decode_weights(packed, n, k)
    sc = layouts.decode_scales(scales, n, k, d.w_group)
    if proj == "gateup":
        codes = layouts.gateup_logical_order(codes, d.intermediate)
        sc = layouts.gateup_logical_order(sc, d.intermediate)
    folded = m if g is None else oracle.fold_gain(m, g)
    want_q, want_s = oracle.quantize_weight_rtn(folded, d.w_group)
    np.testing.assert_array_equal(codes, want_q)
    np.testing.assert_array_equal(sc.view(np.uint16), want_s.view(np.uint16))


def _host_pack_codes(fx, dims, proj, canon, canon_scales):
    pb, sb = fx.futx_packed_sizes(dims, proj)
    packed = np.zeros(pb, np.uint8)
    scales = np.zeros(sb // 2, np.uint16)
    fx.futx_pack_codes_host(dims, proj, canon, canon_scales, packed, scales)
    return packed, scales


@pytest.mark.parametrize("proj", ["qkv", "o", "gateup", "down"])
def test_pack_codes_equals_rtn_pack(fx, proj):
    """Codes and scales quantized outside the library (here: the oracle's
    round-to-nearest) enter through futx_pack_codes_host and give exactly
    the device bytes of futx_pack_weights_host on the same weights."""
    wl = W.tiny()
    w = W.block_weights(wl, 0)
    d = wl.dims
    mats = {"qkv": (w["wqkv"], w["gain_attn"]), "o": (w["wo"], None),
            "gateup": (np.concatenate([w["wgate"], w["wup"]]), w["gain_ffn"]), "down": (w["wdown"], None)}
    m, g = mats[proj]
    folded = m if g is None else oracle.fold_gain(m, g)
    q, s = oracle.quantize_weight_rtn(folded, d.w_group)
    got_p, got_s = _host_pack_codes(fx, d, proj, oracle.pack_nibbles(q), s.view(np.uint16))
    want_p, want_s = _host_pack(fx, d, proj, m, g)
    np.testing.assert_array_equal(got_p, want_p)
    np.testing.assert_array_equal(got_s, want_s)


@pytest.mark.parametrize("proj", ["qkv", "gateup", "down"])
def test_pack_codes_full_code_range(fx, proj):
    """Every code in [-8, 7] (-8 never comes out of max/7 round-to-nearest,
    but external quantizers may use it) and arbitrary finite scales survive
    the reorder, read back by the independent layout decoder."""
    d = W.TINY
    r = np.random.default_rng(31)
    pb, _ = fx.futx_packed_sizes(d, proj)
    n, k = {"qkv": (512, 256), "gateup": (1536, 256), "down": (256, 768)}[proj]
    q = r.integers(-8, 8, (n, k)).astype(np.int8)
    q[0, :16] = np.arange(-8, 8)
    s = (r.standard_normal((n, k // d.w_group)) * 0.01).astype(np.float16)
    packed, scales = _host_pack_codes(fx, d, proj, oracle.pack_nibbles(q), s.view(np.uint16))
    codes = layouts.decode_weights(packed, n, k)
    sc = layouts.decode_scales(scales, n, k, d.w_group)
    if proj == "gateup":
        codes = layouts.gateup_logical_order(codes, d.intermediate)
        sc = layouts.gateup_logical_order(sc, d.intermediate)
    np.testing.assert_array_equal(codes, q)
    np.testing.assert_array_equal(sc.view(np.uint16), s.view(np.uint16))


def test_pack_codes_rejects_non_finite_scale(fx):
    d = W.TINY
    n, k = 256, 768
    s = np.full((n, k // d.w_group), 0.01, np.float16)
    s[3, 2] = np.inf
    with pytest.raises(fx.FutxError) as e:
        _host_pack_codes(fx, d, "down", np.zeros((n, k // 2), np.uint8), s.view(np.uint16))
    assert e.value.status == fx.FUTX_E_RANGE


def test_pack_codes_rejects_null_and_bad_projection(fx):
    d = W.TINY
    pb, sb = fx.futx_packed_sizes(d, "down")
    packed, scales = np.zeros(pb, np.uint8), np.zeros(sb // 2, np.uint16)
    sc = np.zeros((256, 12), np.uint16)
    # null codes pointer, through the C entry point directly
    st = fx._lib.futx_pack_codes_host(fx.ctypes.byref(fx.make_dims(d)), fx.FUTX_PROJ_DOWN, None, fx._ptr(sc),
                                      fx._ptr(packed), fx._ptr(scales))
    assert st == fx.FUTX_E_ARG
    with pytest.raises(fx.FutxError) as e:
        fx._check("futx_pack_codes_host", fx._lib.futx_pack_codes_host(
            fx.ctypes.byref(fx.make_dims(d)), 7, None, None, None, None))
    assert e.value.status == fx.FUTX_E_ARG


def test_host_pack_edge_values(fx):
    """Ties, zero groups, fp16-subnormal scales, the -8 code from external
    codes cannot arise; large but representable scales."""
    d = W.TINY
    r = np.random.default_rng(11)
    w = (r.standard_normal((256, 256)) * 0.02).astype(np.float32)
    w[0, :64] = 0.0
    w[1, :64] = np.float32(1e-6) * r.standard_normal(64).astype(np.float32)  # subnormal fp16 scale
    w[2, :64] = np.float32(1e-9)  # rounds to a zero scale
    w[3, :8] = [7, 3.5, -2.5, 0.5, 0, 0, 0, 0]
    w[4, :64] = np.float32(4.0e5)  # scale 57142.86 (fp16-representable range)
    w[5, :64] = np.linspace(-1, 1, 64, dtype=np.float32)
    packed, scales = _host_pack(fx, d, "o", w, None)
    codes = layouts.decode_weights(packed, 256, 256)
    want_q, want_s = oracle.quantize_weight_rtn(w, 64)
    np.testing.assert_array_equal(codes, want_q)
    np.testing.assert_array_equal(layouts.decode_scales(scales, 256, 256, 64).view(np.uint16), want_s.view(np.uint16))
    w[6, 0] = np.float32(1e6)  # max|w|/7 overflows fp16
    with pytest.raises(fx.FutxError) as e:
        _host_pack(fx, d, "o", w, None)
    assert e.value.status == fx.FUTX_E_RANGE


def test_host_pack_bit_exact_8b_slice(fx):
    """A full-width 8B-shape O projection (K = 4096, group 128)."""
    wl = W.llama8b()
    r = np.random.default_rng(12)
    w = (r.standard_normal((4096, 4096)) * 0.02).astype(np.float32)
    packed, scales = _host_pack(fx, wl.dims, "o", w, None)
    codes = layouts.decode_weights(packed, 4096, 4096)
    want_q, want_s = oracle.quantize_weight_rtn(w, 128)
    np.testing.assert_array_equal(codes, want_q)
    np.testing.assert_array_equal(layouts.decode_scales(scales, 4096, 4096, 128).view(np.uint16), want_s.view(np.uint16))


def test_fold_head_matches_oracle(fx):
    r = np.random.default_rng(13)
    vocab, hidden = 300, 256
    w = W.to_bf16_values((r.standard_normal((vocab, hidden)) * 0.02).astype(np.float32))
    gain = r.uniform(0.5, 1.5, hidden).astype(np.float32)
    wbits = (w.view(np.uint32) >> 16).astype(np.uint16)
    out = np.zeros((vocab, hidden), np.uint16)
    fx.futx_fold_head(vocab, hidden, wbits, gain, out)
    got = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(got, oracle.fold_head(w, gain))


def test_head_tables_round_to_nearest_even():
    """DecodeHead's fp32 -> bf16 conversion rounds to nearest even (torch's
    cast), so tables that are not already bf16-valued are not truncated."""
    torch = pytest.importorskip("torch")
    from int4_weight_kv_amd.block import bf16_bits

    r = np.random.default_rng(3)
    ties = ((r.integers(0x3F000000, 0x40800000, 4000, dtype=np.uint32) & 0xFFFF0000) | 0x8000).view(np.float32)
    x = np.concatenate([r.standard_normal(50000).astype(np.float32), ties,
                        np.array([np.inf, -np.inf, 0.0, -0.0, 3.0e38, 1e-40], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_bits(x), want)
