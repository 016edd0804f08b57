"""GPU parity of the FP8 (e4m3) projection.

* futx_fp8_quantize_act: codes and scales equal the oracle's recipe bit for
  bit (IEEE fp32 division on both sides), on rows with a wide dynamic range
  (subnormal codes), all-zero and single-entry groups, negative zeros and
  hand-placed rounding ties.
* futx_fp8_linear, exact-product case: every weight and activation code has
  the top exponent (|x| within [0.6, 1] of its group's maximum), so each
  group sum on the fp8 matrix cores is exact (all products are multiples of
  2^10 below 2^25) and the output must equal the oracle's fp64 product to
  the fp32 scaling and summation error alone: (K/128 + 8) 2^-24 sum|terms|.
  A wrong scale, group or row anywhere misses this by orders of magnitude.
* futx_fp8_linear, realistic data: the gfx950 fp8 instruction truncates
  each product toward zero to a grid of 2^(E_r - 13), where E_r is the
  largest sum of the two operands' exponent fields (subnormal codes count
  as -6, the mantissa carry does not) over the run r of 8 consecutive
  inputs it sits in; the run sums are then combined on a finer grid
  (measured on the device: a 2^-13 product beside 1.0 survives, a 2^-14
  one does not; a run sum 2^-18 below the largest survives).  Bound per
  output: sum over groups |s_w s_a| sum over runs 12 2^(E_r - 13) (at most
  8 truncated products per run plus 4 for the combination of the 4 runs of
  one instruction) plus the fp32 term above.  Checked with the exact E_r on
  sampled columns and with E_r <= max exponent of a + max exponent of w on
  every column.
"""

import numpy as np
import pytest

from oracle import fp8
from int4_weight_kv_amd import workload as W

from .gpu_common import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

GROUP = 128
RUN = 8


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from int4_weight_kv_amd import futx

    return futx


def _bf16_bits(x32):
    return (np.ascontiguousarray(x32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _exp_field(codes):
    """Exponent of an e4m3 code as the matrix instruction aligns it: field - 7,
    subnormals (field 0, zero included) at -6."""
    f = ((np.asarray(codes, np.uint8) >> 3) & 15).astype(np.int64)
    return np.where(f == 0, -6, f - 7)


def _terms(a_codes, a_scales, w_codes, w_scales):
    """|s_w s_a| sum |w a| per (b, n), fp64."""
    av = np.abs(fp8.dequant_groups(a_codes, a_scales))
    wv = np.abs(fp8.dequant_groups(w_codes, w_scales))
    return av @ wv.T


def _trunc_bound_sampled(a_codes, a_scales, w_codes, w_scales, cols):
    """sum_g |s_w s_a| sum_r 12 2^(E_r - 13) with the exact run exponent, for columns `cols`."""
    ea = _exp_field(a_codes)                  # [B, K]
    ew = _exp_field(w_codes[cols])            # [C, K]
    B, K = ea.shape
    e = ea[:, None, :] + ew[None, :, :]       # [B, C, K]
    er = e.reshape(B, len(cols), K // RUN, RUN).max(axis=-1)  # [B, C, R]
    per_group = (12.0 * np.exp2(er - 13.0)).reshape(B, len(cols), K // GROUP, GROUP // RUN).sum(axis=-1)
    s = np.abs(a_scales.astype(np.float64))[:, None, :] * np.abs(w_scales[cols].astype(np.float64))[None, :, :]
    return (per_group * s).sum(axis=-1)


def _trunc_bound_all(a_codes, a_scales, w_codes, w_scales):
    """The same with E_r replaced by (max exponent of a over r) + (max exponent of w over r): every column."""
    B, K = a_codes.shape
    N = w_codes.shape[0]
    ma = _exp_field(a_codes).reshape(B, K // RUN, RUN).max(axis=-1)
    mw = _exp_field(w_codes).reshape(N, K // RUN, RUN).max(axis=-1)
    sa = np.repeat(np.abs(a_scales.astype(np.float64)), GROUP // RUN, axis=-1)
    sw = np.repeat(np.abs(w_scales.astype(np.float64)), GROUP // RUN, axis=-1)
    return 12.0 * ((np.exp2(ma - 13.0) * sa) @ (np.exp2(mw.astype(np.float64)) * sw).T)


def _run_linear(F, d, proj, m, g, act):
    from int4_weight_kv_amd import block as DB

    batch = act.shape[0]
    n = m.shape[0]
    pb, sb = F.futx_fp8_packed_sizes(d, proj)
    packed, scales = DB.device_buffer(pb), DB.device_buffer(sb)
    F.futx_pack_fp8_weights(d, proj, m, g, packed, scales)
    ws_bytes = F.futx_fp8_linear_workspace_size(d, proj, batch)
    ws = DB.device_buffer(ws_bytes)
    out = torch.empty((batch, n), dtype=torch.float32, device="cuda")
    F.futx_fp8_linear(d, proj, (packed, scales), batch, torch.from_numpy(_bf16_bits(act)).cuda(), out, ws, ws_bytes)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _quant_rows(r, rows, k):
    x = (r.standard_normal((rows, k)) * np.exp(3.0 * r.standard_normal((rows, k)))).astype(np.float32)
    x = W.to_bf16_values(x)
    x[0, :GROUP] = 0.0                                  # all-zero group
    if k >= 2 * GROUP:
        x[0, GROUP:2 * GROUP] = 0.0
        x[0, GROUP + 5] = -3.0                          # a single entry (negative)
    if rows > 1:
        x[1, :GROUP] = np.float32(-0.0)                 # negative zeros
        # group maximum 448 (s = 1): ties at 17, 19, 2^-10, 3 2^-10 and 232
        x[1, 0] = 448.0
        x[1, 1:9] = [17.0, 19.0, -17.0, 2.0 ** -10, 3 * 2.0 ** -10, 232.0, -240.0, 0.75 * 2.0 ** -6]
    return W.to_bf16_values(x)


@pytest.mark.parametrize("rows,k", [(1, 128), (7, 256), (33, 4096), (5, 14336)])
def test_fp8_quantize_act_bit_exact(F, rows, k):
    r = np.random.default_rng(70 + rows)
    x = _quant_rows(r, rows, k)
    codes = torch.empty((rows, k), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, k // GROUP), dtype=torch.float32, device="cuda")
    say("fp8_quantize_act rows %d k %d" % (rows, k))
    F.futx_fp8_quantize_act(k, rows, torch.from_numpy(_bf16_bits(x)).cuda(), codes, scales)
    torch.cuda.synchronize()
    want_c, want_s = fp8.quantize_groups(x)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32))
    bad = np.flatnonzero(got_c != want_c)
    assert bad.size == 0, ("codes differ", bad[:8], got_c.ravel()[bad[:8]], want_c.ravel()[bad[:8]])
    # the hand-placed cases decode as the recipe says (s = 1 for row 1 group 0)
    if rows > 1:
        assert list(want_c[1, 1:9]) == [0x58, 0x5A, 0xD8, 0x00, 0x02, 0x76, 0xF7, 0x06]


def _top_exponent(r, shape, mag):
    """|x| in [0.6, 1] of `mag` (per row) with random signs and one entry per
    group at exactly `mag`: every e4m3 code of the group then has exponent 8."""
    u = r.uniform(0.6, 1.0, shape) * np.where(r.random(shape) < 0.5, -1.0, 1.0)
    u.reshape(shape[:-1] + (shape[-1] // GROUP, GROUP))[..., 0] = 1.0
    return (u * mag).astype(np.float32)


@pytest.mark.parametrize("shape", ["tiny", "8b"])
@pytest.mark.parametrize("batch", [1, 17, 32])
def test_fp8_linear_exact_products(F, shape, batch):
    wl = W.tiny() if shape == "tiny" else W.llama8b()
    d = wl.dims
    r = np.random.default_rng(80 + batch)
    for proj in ("qkv", "o", "gateup", "down"):
        if shape == "8b" and proj != ("down" if batch == 32 else "qkv"):
            continue
        w = W.block_weights(wl, 0)
        n, k = {"qkv": w["wqkv"].shape, "o": w["wo"].shape, "down": w["wdown"].shape,
                "gateup": (2 * w["wgate"].shape[0], w["wgate"].shape[1])}[proj]
        m = _top_exponent(r, (n, k), np.exp(r.standard_normal((n, 1))) * 0.05)
        act = W.to_bf16_values(_top_exponent(r, (batch, k), np.exp(r.standard_normal((batch, 1)))))
        if batch > 1:
            act[1, :GROUP] = 0.0
        wc, wsc = fp8.quantize_groups(m)
        ac, asc = fp8.quantize_groups(act)
        live = np.any(ac != 0, axis=1)
        assert np.all(_exp_field(ac[live][ac[live] != 0]) == 8) and np.all(_exp_field(wc) == 8)
        say("fp8_linear exact products", shape, proj, "batch", batch)
        got = _run_linear(F, d, proj, m, None, act)
        ref = fp8.fp8_linear(act, wc, wsc)
        bound = (k // GROUP + 8) * 2.0 ** -24 * _terms(ac, asc, wc, wsc) + 1e-30
        ratio = float(np.max(np.abs(got - ref) / bound))
        say("  max err / bound %.3g (max|ref| %.3g)" % (ratio, float(np.max(np.abs(ref)))))
        assert ratio <= 1.0, (proj, ratio)


@pytest.mark.parametrize("shape", ["tiny", "8b"])
@pytest.mark.parametrize("batch", [1, 5, 16, 17, 32])
def test_fp8_linear(F, shape, batch):
    wl = W.tiny() if shape == "tiny" else W.llama8b()
    w = W.block_weights(wl, 0)
    r = np.random.default_rng(60 + batch)
    for proj, m, g in (("qkv", w["wqkv"], w["gain_attn"]), ("o", w["wo"], None),
                       ("gateup", np.concatenate([w["wgate"], w["wup"]]), w["gain_ffn"]), ("down", w["wdown"], None)):
        if shape == "8b" and proj in ("qkv", "o") and batch not in (1, 32):
            continue
        n, k = m.shape
        act = W.to_bf16_values((r.standard_normal((batch, k)) * np.exp(r.standard_normal((batch, 1)))).astype(np.float32))
        if batch > 1:
            act[1, :GROUP] = 0.0  # an all-zero activation group
        say("fp8_linear", shape, proj, "batch", batch)
        got = _run_linear(F, wl.dims, proj, m, g, act)
        folded = m if g is None else (m * g[None, :]).astype(np.float32)
        wc, wsc = fp8.quantize_groups(folded)
        ac, asc = fp8.quantize_groups(act)
        ref = fp8.fp8_linear(act, wc, wsc)
        err = np.abs(got - ref)
        fp32_term = (k // GROUP + 12) * 2.0 ** -24 * _terms(ac, asc, wc, wsc)
        bound_all = _trunc_bound_all(ac, asc, wc, wsc) + fp32_term + 1e-30
        cols = np.unique(np.concatenate([[0, n - 1], r.choice(n, min(n, 48), replace=False)]))
        bound_cols = _trunc_bound_sampled(ac, asc, wc, wsc, cols) + fp32_term[:, cols] + 1e-30
        r_all = float(np.max(err / bound_all))
        r_cols = float(np.max(err[:, cols] / bound_cols))
        say("  max err %.3g (max|ref| %.3g); err / bound: every column %.3g, sampled columns %.3g"
            % (float(err.max()), float(np.max(np.abs(ref))), r_all, r_cols))
        assert r_all <= 1.0 and r_cols <= 1.0, (proj, r_all, r_cols)
