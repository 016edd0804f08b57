"""Rounding helpers of the oracle (test infrastructure only).

bf16_round
    Rounds fp64 values to the nearest bfloat16 value, ties to even, in ONE
    rounding step (no detour through fp32).  bfloat16 has 8 significant bits
    and fp32's exponent range (normal numbers down to 2**-126, subnormals down
    to 2**-133).  The pages fix no rounding mode; round-to-nearest-even is the
    IEEE default and what the matrix-core operand conversion on the GPU uses.
    Pinned by tests against torch's float32->bfloat16 conversion (a library
    routine) on every fp32-representable input, including ties and
    subnormals.

fp16_round_from_fp32
    IEEE binary16 round-to-nearest-even of fp32 values, via numpy's cast (a
    library routine).  Used for every stored scale.
"""

import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")  # (2 - 2**-7) * 2**127


def bf16_round(x):
    """Nearest bfloat16 value of each element of ``x`` (ties to even), as fp64."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    nz = np.isfinite(x) & (x != 0.0)
    v = x[nz]
    _, e = np.frexp(v)  # v = m * 2**e with 0.5 <= |m| < 1
    # bfloat16 spacing at this magnitude is 2**(e - 8); below the normal range
    # the spacing stays at the subnormal step 2**-133.
    e_sp = np.maximum(e - 8, -133)
    q = np.rint(np.ldexp(v, -e_sp))  # exact power-of-two scaling, then RNE
    r = np.ldexp(q, e_sp)
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)
    out[nz] = r
    return out


def fp16_round_from_fp32(x32):
    """IEEE half precision of fp32 input, round to nearest even (numpy cast)."""
    x32 = np.asarray(x32, dtype=np.float32)
    return x32.astype(np.float16)
