"""Rotary position embedding (oracle, test infrastructure only).

The pages describe a "Llama-style" Transformer block [ABS] and say nothing
else about positions.  Reading: the rotate-half RoPE convention of the
Hugging Face Llama implementation (the compiled ``transformers`` step is the
pages' baseline), pairs (i, i + d/2) for i < d/2, frequency theta**(-2i/d),
no frequency scaling, angle p * theta_i computed in fp64.

    (a, b) -> (a cos(p th_i) - b sin(p th_i),  b cos(p th_i) + a sin(p th_i))
    with a = x[i], b = x[i + d/2]

Pins (tests/test_oracle_pins.py, tests/golden/rope_cases.txt): p = 0 is the
identity; pair norms are
preserved; (R_m q).(R_n k) depends on m - n only; a hand-computed d = 4 case.
"""

import numpy as np


def rope_inv_freq(d, theta):
    """theta**(-2i/d) for i = 0 .. d/2 - 1, fp64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / np.float64(d))


def rope_rotate_half(x, pos, theta):
    """Rotate the last axis (size d) of ``x`` at integer position(s) ``pos``.

    ``pos`` broadcasts against ``x.shape[:-1]``.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("head_dim must be even")
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., : d // 2], x[..., d // 2 :]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
