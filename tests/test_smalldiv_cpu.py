"""The GEMM kernel's division by a runtime divisor (SmallDiv in
int4_weight_kv_amd/csrc/gemm.hip): q = trunc(fp32(x) * r) with r the fp32
reciprocal of d, then one correction down and one up.  The device reciprocal
is within 1 ulp of 1/d, so this checks the argument with r rounded to nearest
and moved one ulp either way: for every dividend below 2^20 the result must
equal floor(x / d).  The steps are the same fp32 operations the kernel
issues (convert, multiply, truncate, two integer corrections)."""

import numpy as np
import pytest

X = np.arange(1 << 20, dtype=np.int64)
XF = X.astype(np.float32)


def _small_div(x, xf, d, r):
    q = (xf * np.float32(r)).astype(np.float32).astype(np.int64)  # truncation toward zero
    q -= (q * d > x).astype(np.int64)
    q += ((q + 1) * d <= x).astype(np.int64)
    return q


def _reciprocals(d):
    r = np.float32(1.0) / np.float32(d)
    return (np.nextafter(r, np.float32(0)), r, np.nextafter(r, np.float32(np.inf)))


DIVISORS = list(range(1, 161)) + [191, 255, 256, 257, 509, 1000, 1023, 1024, 4093, 4096, 16381, 65521]


@pytest.mark.parametrize("d", DIVISORS)
def test_small_div_exact_below_2_20(d):
    want = X // d
    for r in _reciprocals(d):
        got = _small_div(X, XF, d, r)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (d, float(r), X[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_small_div_needs_the_correction():
    # without the corrections a one-ulp-low reciprocal truncates exact
    # multiples to one less: the corrections are not dead code
    d = 3
    r = _reciprocals(d)[0]
    raw = (XF * np.float32(r)).astype(np.float32).astype(np.int64)
    assert np.any(raw != X // d)
