"""Block-diagonal Hadamard rotation (oracle, test infrastructure only).

What the pages fix: a block-diagonal Hadamard transform spreads the energy
of outlier channels before the KV cache is quantized to INT4 [ABS]; it is an
orthogonal transform, applied on the way into the cache and undone on the
way out [INT4, Hadamard explainer paragraph].

Readings: Sylvester construction in natural order, H_n[i][j] =
(-1)**popcount(i & j), normalized by 1/sqrt(n) so that it is orthogonal,
symmetric and its own inverse; no random signs; the blocks are contiguous
runs of ``hb`` channels of one head (hb = 32 or 64).

Pins (tests/test_oracle_pins.py, tests/golden/hadamard_cases.txt): H H^T =
n I exactly in integers for
n = 32 and 64; equality with scipy.linalg.hadamard (a library routine);
symmetry and involution of the normalized matrix; the hand value
Hn_64 (16 e_0) = (2, ..., 2); invariance of dot products under the same
block rotation of both operands.
"""

import numpy as np


def sylvester(n):
    """Integer Sylvester Hadamard matrix of order ``n`` (a power of two)."""
    if n < 1 or n & (n - 1):
        raise ValueError("Hadamard order must be a power of two")
    i = np.arange(n)
    bits = np.bitwise_and(i[:, None], i[None, :])
    parity = np.zeros((n, n), dtype=np.int64)
    while np.any(bits):
        parity ^= bits & 1
        bits >>= 1
    return (1 - 2 * parity).astype(np.int64)


def hadamard_normalized(n):
    """H_n / sqrt(n) in fp64."""
    return sylvester(n).astype(np.float64) / np.sqrt(np.float64(n))


def block_diag_rotate(x, hb):
    """Apply the normalized Hadamard to each contiguous block of ``hb`` entries
    of the last axis of ``x`` (fp64 dense matmul per block)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % hb:
        raise ValueError("head_dim must be a multiple of the Hadamard block")
    h = hadamard_normalized(hb)
    xb = x.reshape(x.shape[:-1] + (d // hb, hb))
    yb = xb @ h.T
    return yb.reshape(x.shape)
