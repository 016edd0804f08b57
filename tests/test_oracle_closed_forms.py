"""Closed-form pins of the oracle's composed steps: RMSNorm scaling inside the
block (O4/O5, O11/O12), the LM head (O15 tail), the head fold, the gain fold
and the full step (O15), each against values fixed by mathematics rather than
by the oracle's own formulas:

* a constant row x = c 1 makes the norm's operand bf16(c) 1 and its scale
  sqrt(c^2 + eps), so every projection output is bf16(c) times a row sum of
  the dequantized weights over that scale;
* with the O-projection codes all zero the attention path adds nothing, so
  h = x and the MLP input is the block input;
* with eps = 0 the whole norm is invariant under x -> 2^k x (bf16 rounding
  commutes with powers of two);
* a head whose row v is the unit vector e_(v mod H) returns x[v mod H] / r,
  with ties among rows v = j, j + H, ... resolved to the lowest index;
* zero projection weights make every block the identity, so the full step
  reduces to the head applied to the embedding row;
* power-of-two gains fold without rounding: codes unchanged, scales x 2^k.

Planted mistakes at the end check that these pins catch the slips that the
composed-block sanity test cannot see (dropping 1/r, a wrong eps, a wrong
argmax index)."""

import math

import numpy as np
import pytest

import oracle
from oracle import block as oblock

TINY = oracle.BlockDims(256, 4, 2, 64, 768, 64, 32)


def _bf16(v):
    """bf16 of a scalar via torch's cast (a library routine), as float."""
    torch = pytest.importorskip("torch")
    return float(torch.tensor([v], dtype=torch.float64).to(torch.float32).to(torch.bfloat16).to(torch.float64)[0])


def _random_weights(dims, rng, zero_o=False):
    """QuantBlockWeights from random codes and fp16 scales (no quantizer
    involved); the dense matrices are codes * scales, written here by hand."""
    g = dims.w_group
    shapes = {
        "qkv": (dims.n_qkv, dims.hidden),
        "o": (dims.hidden, dims.n_heads * dims.head_dim),
        "gate": (dims.intermediate, dims.hidden),
        "up": (dims.intermediate, dims.hidden),
        "down": (dims.hidden, dims.intermediate),
    }
    codes, scales, dense = {}, {}, {}
    for name, (n, k) in shapes.items():
        c = rng.integers(-8, 8, (n, k)).astype(np.int8)
        s = (rng.uniform(0.5, 1.5, (n, k // g)) * 0.01).astype(np.float16)
        if name == "o" and zero_o:
            c[:] = 0
        codes[name], scales[name] = c, s
        dense[name] = c.astype(np.float64) * np.repeat(s.astype(np.float64), g, axis=1)
    return oracle.QuantBlockWeights(group=g, codes=codes, scales=scales), dense


def _caches(dims, lens, rng):
    out = []
    for L in lens:
        c = oracle.LogicalKVCache.empty(L + 1, dims.n_kv_heads, dims.head_dim)
        if L:
            k = rng.standard_normal((L, dims.n_kv_heads, dims.head_dim)).astype(np.float32)
            v = rng.standard_normal((L, dims.n_kv_heads, dims.head_dim)).astype(np.float32)
            oracle.history_fill(c, k, v, np.arange(L), dims)
        out.append(c)
    return out


# constants whose bf16 rounding is visible (1 + 2^-10 rounds to 1), a
# negative row, and a small row where eps is 10% of the mean square
CONSTS = [1.0 + 2.0 ** -10, -3.3, 0.01]


def test_qkv_closed_form_constant_row():
    """O4/O5: x = c 1 -> qkv = bf16(c) rowsum(W_qkv) / sqrt(c^2 + eps)."""
    rng = np.random.default_rng(100)
    qw, dense = _random_weights(TINY, rng)
    x = np.array([[c] * TINY.hidden for c in CONSTS], np.float32)
    diag = {}
    oracle.decode_block(x, qw, _caches(TINY, [5, 0, 70], rng), np.array([5, 0, 70]), TINY, diag=diag)
    rs = dense["qkv"].sum(axis=1)
    for b, c in enumerate(CONSTS):
        c32 = float(np.float32(c))
        want = _bf16(c32) * rs / math.sqrt(c32 * c32 + TINY.rms_eps)
        np.testing.assert_allclose(diag["qkv"][b], want, rtol=1e-12, atol=1e-300)


def test_mlp_closed_form_with_silent_attention():
    """O10-O13 with the O-projection codes all zero: h = x, then
    g = bf16(c) rowsum(W_gate) / sqrt(c^2 + eps), likewise up, and
    y = x + W_down bf16(silu(g) up)."""
    rng = np.random.default_rng(101)
    qw, dense = _random_weights(TINY, rng, zero_o=True)
    x = np.array([[c] * TINY.hidden for c in CONSTS], np.float32)
    diag = {}
    y = oracle.decode_block(x, qw, _caches(TINY, [3, 64, 1], rng), np.array([3, 64, 1]), TINY, diag=diag)
    np.testing.assert_array_equal(diag["h"], x.astype(np.float64))
    rg, ru = dense["gate"].sum(axis=1), dense["up"].sum(axis=1)
    for b, c in enumerate(CONSTS):
        c32 = float(np.float32(c))
        r2 = math.sqrt(c32 * c32 + TINY.rms_eps)
        g = _bf16(c32) * rg / r2
        up = _bf16(c32) * ru / r2
        np.testing.assert_allclose(diag["g"][b], g, rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(diag["up"][b], up, rtol=1e-12, atol=1e-300)
        # act is the bf16 value next to silu(g) up: representable in bf16 and
        # within half a bf16 step (2^-8 relative: 8 significant bits) of it
        z = g / (1.0 + np.exp(-g)) * up
        act = diag["act"][b]
        np.testing.assert_array_equal(act, [_bf16(float(a)) for a in act.astype(np.float32)])
        assert np.all(np.abs(act - z) <= 2.0 ** -8 * np.abs(z) + 1e-300)
        np.testing.assert_allclose(y[b], c32 + dense["down"] @ act, rtol=1e-12, atol=1e-12)


def test_norm_scale_invariance():
    """With eps = 0, x -> 2^k x leaves qkv unchanged (and g, up when the
    attention path is silent), for k = 3 and k = -4: a block that forgot to
    divide by r would scale them by 2^k."""
    rng = np.random.default_rng(102)
    dims = oracle.BlockDims(256, 4, 2, 64, 768, 64, 32, rms_eps=0.0)
    qw, _ = _random_weights(dims, rng, zero_o=True)
    x = (rng.standard_normal((2, dims.hidden)) * 1.7).astype(np.float32)
    lens = np.array([9, 40])
    base = {}
    oracle.decode_block(x, qw, _caches(dims, lens, np.random.default_rng(7)), lens, dims, diag=base)
    for k in (3, -4):
        d = {}
        oracle.decode_block(np.ldexp(x, k).astype(np.float32), qw, _caches(dims, lens, np.random.default_rng(7)),
                            lens, dims, diag=d)
        for name in ("qkv", "g", "up"):
            np.testing.assert_allclose(d[name], base[name], rtol=1e-12, atol=1e-300, err_msg=name)


def _unit_head(vocab, hidden):
    w = np.zeros((vocab, hidden))
    w[np.arange(vocab), np.arange(vocab) % hidden] = 1.0
    return w


def test_lm_head_unit_rows_and_lowest_index_ties():
    """O15 tail: rows e_(v mod H) give logits[v] = bf16(x[v mod H]) / r, with
    r = sqrt(mean(x^2) + eps); the maximum repeats at j, j + H, j + 2H and the
    top-1 is the lowest of them."""
    hidden, vocab, eps = 64, 3 * 64 + 17, 1e-5
    rng = np.random.default_rng(103)
    x = (rng.standard_normal((3, hidden)) * np.array([[1.0], [0.01], [5.0]])).astype(np.float32)
    logits, top1 = oracle.lm_head(x, _unit_head(vocab, hidden), eps)
    for b in range(3):
        xb = x[b].astype(np.float64)
        r = math.sqrt(float(np.sum(xb * xb)) / hidden + eps)
        want = np.array([_bf16(float(x[b, v % hidden])) for v in range(vocab)]) / r
        np.testing.assert_allclose(logits[b], want, rtol=1e-13, atol=0)
        ub = np.array([_bf16(float(t)) for t in x[b]])
        j = int(np.argmax(ub))
        assert np.sum(ub == ub[j]) == 1  # unique largest channel
        assert int(top1[b]) == j, (b, int(top1[b]), j)


def test_fold_head_powers_of_two():
    """bf16(fp32(W * 2^k)) = 2^k W exactly for bf16 W; a general gain matches
    torch's fp32 product rounded to bf16."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(104)
    w = torch.from_numpy(rng.standard_normal((40, 32)).astype(np.float32)).to(torch.bfloat16).to(torch.float32)
    w = w.numpy()
    e = rng.integers(-3, 4, 32)
    gain = np.ldexp(np.ones(32), e).astype(np.float32)
    np.testing.assert_array_equal(oracle.fold_head(w, gain), w.astype(np.float64) * gain[None, :])
    gain2 = rng.uniform(0.5, 1.5, 32).astype(np.float32)
    want = (torch.from_numpy(w) * torch.from_numpy(gain2)[None, :]).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.fold_head(w, gain2), want)


def test_fold_gain_powers_of_two_per_group():
    """Gains that are a power of two per quantization group fold exactly: the
    codes equal those of the unfolded weights and each group's scale is
    multiplied by that group's power of two (a square matrix, so folding the
    wrong axis would scale rows instead and fail)."""
    rng = np.random.default_rng(105)
    g = 64
    w = (rng.standard_normal((256, 256)) * 0.02).astype(np.float32)
    e = rng.integers(-2, 3, 256 // g)
    gain = np.repeat(np.ldexp(np.ones(256 // g), e), g).astype(np.float32)
    q0, s0 = oracle.quantize_weight_rtn(w, g)
    q1, s1 = oracle.quantize_weight_rtn(oracle.fold_gain(w, gain), g)
    np.testing.assert_array_equal(q1, q0)
    np.testing.assert_array_equal(s1.astype(np.float64), s0.astype(np.float64) * np.ldexp(1.0, e)[None, :])


def test_decode_step_identity_layers():
    """O15: with every projection zero, each block returns its input (the
    attention output is multiplied by zero O weights; gate and up are zero),
    so the step's logits are the head applied to the embedding rows:
    logits[b][v] = Emb[tok_b][v mod H] / sqrt(mean(Emb[tok_b]^2) + eps)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(106)
    dims = TINY
    vocab = 300
    emb = torch.from_numpy(rng.standard_normal((vocab, dims.hidden)).astype(np.float32) * 0.5)
    emb = emb.to(torch.bfloat16).to(torch.float32).numpy()
    qw, _ = _random_weights(dims, rng)
    for name in qw.codes:
        qw.codes[name][:] = 0
    qw.drop_dense()
    toks = np.array([7, 299, 0])
    lens = np.array([4, 0, 65])
    caches = [_caches(dims, lens, np.random.default_rng(8 + i)) for i in range(2)]
    seen = []
    logits, top1 = oracle.decode_step(toks, emb, 2, lambda l: qw, lambda l: caches[l], lens, dims,
                                      _unit_head(vocab, dims.hidden), progress=seen.append)
    assert seen == [0, 1]
    for b, t in enumerate(toks):
        e = emb[t].astype(np.float64)
        r = math.sqrt(float(np.sum(e * e)) / dims.hidden + dims.rms_eps)
        np.testing.assert_allclose(logits[b], e[np.arange(vocab) % dims.hidden] / r, rtol=1e-13, atol=0)
        assert int(top1[b]) == int(np.argmax(e)), b


# ------------------------------------------------------------ planted mistakes


def _planted_block(monkeypatch, drop):
    """decode_block with one division by the RMS scale removed (qkv or mlp)."""
    real = oblock.rmsnorm_stats
    calls = {"n": 0}

    def stats(x, eps):
        calls["n"] += 1
        r = real(x, eps)
        # the first call in decode_block is RMSNorm-1, the second RMSNorm-2
        first = calls["n"] % 2 == 1
        if (drop == "qkv" and first) or (drop == "mlp" and not first):
            return np.ones_like(r)
        return r

    monkeypatch.setattr(oblock, "rmsnorm_stats", stats)


@pytest.mark.parametrize("drop", ["qkv", "mlp"])
def test_planted_dropped_rms_scale_is_caught(monkeypatch, drop):
    _planted_block(monkeypatch, drop)
    if drop == "qkv":
        with pytest.raises(AssertionError):
            test_qkv_closed_form_constant_row()
    else:
        with pytest.raises(AssertionError):
            test_mlp_closed_form_with_silent_attention()
    with pytest.raises(AssertionError):
        test_norm_scale_invariance()


def test_planted_lm_head_eps_is_caught(monkeypatch):
    real = oblock.rmsnorm_stats
    monkeypatch.setattr(oblock, "rmsnorm_stats", lambda x, eps: real(x, eps * 1e4))
    with pytest.raises(AssertionError):
        test_lm_head_unit_rows_and_lowest_index_ties()


def test_planted_lm_head_index_is_caught(monkeypatch):
    real_argmax = np.argmax

    class _NP:
        def __getattr__(self, name):
            return getattr(np, name)

        @staticmethod
        def argmax(a, axis=None):  # argmax over reversed columns (index not mapped back)
            return real_argmax(a[..., ::-1], axis=axis)

    monkeypatch.setattr(oblock, "np", _NP())
    with pytest.raises(AssertionError):
        test_lm_head_unit_rows_and_lowest_index_ties()


def test_planted_decode_step_skips_embedding_row_is_caught(monkeypatch):
    real = oblock.lm_head
    monkeypatch.setattr(oblock, "lm_head", lambda x, w, eps: real(x[::-1].copy(), w, eps))
    with pytest.raises(AssertionError):
        test_decode_step_identity_layers()
