"""FP8 (e4m3) weight-and-activation variant of the decode projection (oracle,
test infrastructure only).

What the pages fix: besides the INT4 decode path, the authors have an FP8
path, and the INT4 decode block is 31-51% faster than it (FuTransformer
abstract, airebao.com item page; kongchang.com/en article, section "INT4
Decode: letting dequantization feed directly into MMA operands").  The pages
give no FP8 format detail.

Readings (documented, used identically by the oracle and the HIP path):

* the 8-bit format is e4m3 in the OCP "fn" variant: 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
  m * 2^-9; the largest finite magnitude is 448 (0x7E); 0x7F / 0xFF are NaN;
  there are no infinities;
* weights and activations are both quantized, one fp32 scale per group of
  128 consecutive input channels (weights: per output row; activations: per
  batch row): s = fp32(max|x| / 448), codes = e4m3(fp32(x / s)) rounded to
  nearest even and saturated at +-448; an all-zero group has s = 0 and
  codes 0 (negative zero keeps its sign bit);
* the product is sum over groups of s_w * s_a * sum_k w_code_k a_code_k,
  exact products accumulated (fp64 here, fp32 on the device).

Pins (tests/test_oracle_fp8.py, tests/golden/fp8_cases.txt): the decode of
all 256 bytes against torch's float8_e4m3fn (a library routine); the
encoder against torch's cast on random, tie and subnormal inputs within
range; hand-derived codes (ties to even, saturation, subnormals, zero);
the round-trip bound (half a step of the code's exponent); the projection
against a dense fp64 product of the decoded codes.
"""

import numpy as np

E4M3_MAX = 448.0
GROUP = 128


def e4m3_decode(codes):
    """fp64 values of e4m3fn bytes (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.ldexp(1.0, e - 10))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(v32):
    """e4m3fn bytes of fp32 values: round to nearest even, saturate at +-448.

    Computed in fp32 with exact power-of-two scalings: for |v| = f * 2^x
    (frexp, f in [0.5, 1)) the code's exponent is E = x - 1 clamped to
    [-6, 8]; q = rint(|v| * 2^(3 - E)) counts steps of 2^(E - 3); q = 16
    carries into the next exponent; q < 8 (only at E = -6) is subnormal."""
    v = np.asarray(v32, np.float32)
    a = np.abs(v).astype(np.float32)
    _, x = np.frexp(a)
    E = np.clip(x.astype(np.int64) - 1, -6, 8)
    q = np.rint(np.ldexp(a, (3 - E).astype(np.int32))).astype(np.int64)
    carry = q >= 16
    E = np.where(carry, E + 1, E)
    q = np.where(carry, q // 2, q)
    sat = (E > 8) | ((E == 8) & (q > 14))
    code = np.where(q >= 8, ((E + 7) << 3) | (q - 8), q)
    code = np.where(sat, 0x7E, code)
    code = code | np.where(np.signbit(v), 0x80, 0)
    return code.astype(np.uint8)


def quantize_groups(x32, group=GROUP):
    """Codes uint8 [..., K] and fp32 scales [..., K // group] of fp32 rows
    x32 [..., K], one scale per group of `group` consecutive entries."""
    x = np.asarray(x32, np.float32)
    k = x.shape[-1]
    if k % group:
        raise ValueError("K must be a multiple of the group")
    g = x.reshape(x.shape[:-1] + (k // group, group))
    a = np.max(np.abs(g), axis=-1)
    s = (a / np.float32(E4M3_MAX)).astype(np.float32)  # IEEE fp32 division
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (g / s[..., None]).astype(np.float32)
    r = np.where(s[..., None] == 0, np.float32(0), r)
    return e4m3_encode(r).reshape(x.shape), s


def dequant_groups(codes, scales, group=GROUP):
    """fp64 values code * scale of grouped codes [..., K]."""
    c = e4m3_decode(codes)
    s = np.repeat(np.asarray(scales, np.float64), group, axis=-1)
    return c * s


def fp8_linear(act32, w_codes, w_scales, group=GROUP):
    """out[b][n] = sum_g s_w[n][g] s_a[b][g] sum_{k in g} w[n][k] a[b][k]
    with the activation rows quantized per group (quantize_groups); fp64."""
    a_codes, a_scales = quantize_groups(act32, group)
    return dequant_groups(a_codes, a_scales, group) @ dequant_groups(w_codes, w_scales, group).T
