"""INT4 quantizers, nibble packing and gain folding (oracle, test infrastructure only).

What the pages fix: decode uses INT4 projection weights [ABS]; the weights are
rounded to nearest (RTN) -- the accuracy section contrasts RTN with GPTQ in
"the same format" [ACC]; the fixed RMSNorm gain is folded into the weights
that follow the norm [FP8]; the KV cache is an INT4 copy [ABS].

Readings (the pages give no format details):

* symmetric INT4, codes in [-8, 7], one scale per group of ``group``
  consecutive input channels (64 or 128), scale = max|w| / 7 stored as fp16;
* the recipe is pinned in fp32 so that GPU and oracle codes agree bit for
  bit: a = max|w| (fp32), s = fp16(fp32(a / 7)), q = rint(fp32(w / s)) with
  the STORED scale as divisor, clamped to [-8, 7]; ties round to even; a zero
  group gets scale 0 and codes 0;
* weight scales that overflow fp16 are an error; KV scales saturate at 65504;
* canonical nibble order: byte i of a row holds code 2i in its low nibble
  and code 2i+1 in its high nibble, two's complement;
* fold first, then quantize: W' = fp32(W * gain[k]), one fp32 multiply.

Pins (tests/test_oracle_pins.py with tests/golden/quant_cases.txt and
tests/golden/pack_cases.txt; tests/test_oracle_closed_forms.py): hand cases
with exact expected codes/scales, the round-trip bound |w - q*s| <= s/2,
packing hand cases and an exhaustive byte round trip; folding with
power-of-two gains per group leaves the codes unchanged and multiplies each
group scale by its power of two.
"""

import numpy as np

from .numerics import fp16_round_from_fp32

FP16_MAX = 65504.0


def _quantize_groups_fp32(g32, saturate):
    """fp32 RTN over the last axis of ``g32``; returns (codes int8, scales fp16)."""
    g32 = np.asarray(g32, dtype=np.float32)
    a = np.max(np.abs(g32), axis=-1)  # exact in fp32
    s32 = (a / np.float32(7.0)).astype(np.float32)  # IEEE fp32 division
    if saturate:
        s32 = np.minimum(s32, np.float32(FP16_MAX))
    s16 = fp16_round_from_fp32(s32)
    if np.any(np.isinf(s16)):
        raise OverflowError("group scale max|w|/7 exceeds the fp16 range")
    sf = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (g32 / sf).astype(np.float32)  # IEEE fp32 division by the stored scale
    q = np.where(sf == 0, np.float32(0), np.clip(np.rint(r), -8, 7))
    return q.astype(np.int8), s16


def quantize_weight_rtn(w32, group):
    """RTN INT4 of a weight matrix ``w32`` fp32 [N][K], groups of ``group`` along K.

    Returns codes int8 [N][K] in [-8, 7] and scales fp16 [N][K // group].
    """
    w32 = np.asarray(w32, dtype=np.float32)
    n, k = w32.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    q, s = _quantize_groups_fp32(w32.reshape(n, k // group, group), saturate=False)
    return q.reshape(n, k), s


def quantize_kv_token(x32):
    """Per-token INT4 of a cache row: ``x32`` fp32 [..., d], one scale over d.

    Returns codes int8 [..., d] and scales fp16 [...].
    """
    return _quantize_groups_fp32(np.asarray(x32, dtype=np.float32), saturate=True)


def dequant_weight(codes, scales, group):
    """fp64 values q * s of grouped codes [N][K] with scales [N][K // group]."""
    codes = np.asarray(codes, dtype=np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=1)
    return codes * s


def pack_nibbles(codes):
    """Canonical bytes [..., K/2] of INT4 codes [..., K]: low nibble = even k."""
    c = np.asarray(codes, dtype=np.int16)
    if np.any(c < -8) or np.any(c > 7):
        raise ValueError("INT4 codes must lie in [-8, 7]")
    lo = c[..., 0::2] & 15
    hi = c[..., 1::2] & 15
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """Inverse of ``pack_nibbles``: bytes [..., K/2] -> codes int8 [..., K]."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo = b & 15
    hi = b >> 4
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def fold_gain(w32, gain32):
    """W' = fp32(W * gain[k]) (the gain multiplies input channel k)."""
    w32 = np.asarray(w32, dtype=np.float32)
    g = np.asarray(gain32, dtype=np.float32)
    return (w32 * g[None, :]).astype(np.float32)
