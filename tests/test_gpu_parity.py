"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

* packing and the KV quantizer (identical fp32 inputs): bit-exact;
* the full cache write (RoPE + rotation in fp32 on the GPU, fp64 in the
  oracle): equal except codes one step apart where the oracle's value sits
  within 1e-3 of a rounding midpoint, and scales one fp16 step apart near an
  fp16 midpoint; such exceptions below 1e-4 of the elements;
* INT4 projections: fp32-accumulation level agreement;
* block outputs: max|gpu - oracle| <= 2e-3 max|oracle| + 1e-3.
"""

import numpy as np
import pytest

import oracle
from int4_weight_kv_amd import workload as W
from tests import layouts
from tests.gpu_common import (BlockCase, DecodedCache, FlipStats, block_tolerance, cache_tokens, flip_tolerant,
                               oracle_history, say)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from int4_weight_kv_amd import futx

    return futx


@pytest.fixture(scope="module")
def DB(F):
    from int4_weight_kv_amd import block

    return block


# ---------------------------------------------------------------- packing


@pytest.mark.parametrize("shape,proj", [("tiny", "qkv"), ("tiny", "gateup"), ("tiny", "down"), ("8b", "o"),
                                        ("8b", "gateup")])
def test_pack_device_bit_exact(F, DB, shape, proj):
    wl = W.tiny() if shape == "tiny" else W.llama8b()
    d = wl.dims
    w = W.block_weights(wl, 0)
    mats = {"qkv": (w["wqkv"], w["gain_attn"]), "o": (w["wo"], None),
            "gateup": (np.concatenate([w["wgate"], w["wup"]]), w["gain_ffn"]), "down": (w["wdown"], None)}
    m, g = mats[proj]
    say("pack", shape, proj, m.shape)
    pp = DB.pack_projection(d, proj, m, g)
    n, k = m.shape
    canon = np.zeros((n, k // 2), np.uint8)
    csc = np.zeros((n, k // d.w_group), np.uint16)
    F.futx_unpack_weights(d, proj, pp.packed, pp.scales, canon, csc)
    folded = m if g is None else oracle.fold_gain(m, g)
    q, s = oracle.quantize_weight_rtn(folded, d.w_group)
    np.testing.assert_array_equal(canon, oracle.pack_nibbles(q))
    np.testing.assert_array_equal(csc, s.view(np.uint16))
    # raw device bytes through the independent layout decoder
    raw = layouts.decode_weights(pp.packed.cpu().numpy(), n, k)
    if proj == "gateup":
        raw = layouts.gateup_logical_order(raw, d.intermediate)
    np.testing.assert_array_equal(raw, q)


# ---------------------------------------------------------------- KV append


_cache_tokens = cache_tokens


@pytest.mark.parametrize("shape", ["tiny", "8b"])
def test_kv_append_quantizer_bit_exact(F, DB, shape):
    """flags = 0: the stored codes and scales equal the oracle's quantizer on
    the same fp32 inputs, bit for bit, including ties and zero rows."""
    wl = W.tiny() if shape == "tiny" else W.llama8b()
    d = wl.dims
    r = np.random.default_rng(21)
    n, num_pages = 300, 9
    k = r.standard_normal((n, d.n_kv_heads, d.head_dim)).astype(np.float32)
    v = (r.standard_normal((n, d.n_kv_heads, d.head_dim)) * 3).astype(np.float32)
    k[0, 0] = 0.0  # zero row -> scale 0, codes 0
    k[1, 0, :8] = [7, 3.5, -2.5, 0.5, 0, 0, 0, 0]  # exact ties
    k[1, 0, 8:] = 0.0
    v[2, :] = np.float32(1e-9)  # rounds to a zero scale
    slots = r.permutation(num_pages * 64)[:n].astype(np.int32)
    cache = DB.DeviceKVCache(d, num_pages)
    say("kv_append flags=0", shape)
    cache.append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), None,
                 torch.from_numpy(slots).cuda(), flags=0)
    torch.cuda.synchronize()
    K, KS, V, VS = _cache_tokens(cache.host_copy(), d, num_pages, slots)
    qk, sk = oracle.quantize_kv_token(k)
    qv, sv = oracle.quantize_kv_token(v)
    np.testing.assert_array_equal(K, qk)
    np.testing.assert_array_equal(V, qv)
    np.testing.assert_array_equal(KS.view(np.uint16), sk.view(np.uint16))
    np.testing.assert_array_equal(VS.view(np.uint16), sv.view(np.uint16))


_flip_tolerant = flip_tolerant


@pytest.mark.parametrize("shape", ["tiny", "8b", "8b-outliers"])
def test_kv_append_full_chain(F, DB, shape):
    """RoPE + block Hadamard + quantization at arbitrary positions."""
    wl = {"tiny": W.tiny(), "8b": W.llama8b(), "8b-outliers": W.llama8b_ragged(1)}[shape]
    d = wl.dims
    n = 700
    k, v = W.history(wl, 0, 0, n)
    r = np.random.default_rng(22)
    pos = r.integers(0, 9000, n).astype(np.int32)
    num_pages = 16
    slots = r.permutation(num_pages * 64)[:n].astype(np.int32)
    cache = DB.DeviceKVCache(d, num_pages)
    say("kv_append rope+hadamard", shape)
    cache.append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(pos).cuda(),
                 torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    K, KS, V, VS = _cache_tokens(cache.host_copy(), d, num_pages, slots)
    kr, vr = oracle.rotate_kv(k.astype(np.float64), v.astype(np.float64), pos[:, None], d)
    fk = _flip_tolerant(K, KS, kr, "keys", max_per_row=1)
    fv = _flip_tolerant(V, VS, vr, "values", max_per_row=1)
    say("boundary decisions: keys", fk, "; values", fv)


def test_kv_append_rotation_ablation(F, DB):
    """The device cache written with and without the block rotation on the
    outlier-key workload: each flag setting matches the oracle's chain, and
    the rotation cuts the key error (the pages' claim; the oracle-only
    version is in test_rotation_ablation.py)."""
    wl = W.llama8b_ragged(1)
    d = wl.dims
    n, num_pages = 512, 8
    k, v = W.history(wl, 0, 0, n)
    pos = np.arange(n, dtype=np.int32)
    k_rope = oracle.rope_rotate_half(k.astype(np.float64), pos[:, None], d.rope_theta)
    v64 = v.astype(np.float64)
    errs = {}
    for rot in (False, True):
        flags = F.FUTX_KV_ROPE | (F.FUTX_KV_HADAMARD if rot else 0)
        cache = DB.DeviceKVCache(d, num_pages)
        say("kv_append ablation, rotation", rot)
        cache.append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(pos).cuda(),
                     torch.from_numpy(pos.copy()).cuda(), flags=flags)
        torch.cuda.synchronize()
        K, KS, V, VS = _cache_tokens(cache.host_copy(), d, num_pages, pos)
        kx = oracle.block_diag_rotate(k_rope, d.had_block) if rot else k_rope
        vx = oracle.block_diag_rotate(v64, d.had_block) if rot else v64
        _flip_tolerant(K, KS, kx, "keys")
        _flip_tolerant(V, VS, vx, "values")
        kh = K.astype(np.float64) * KS.astype(np.float64)[..., None]
        if rot:
            kh = oracle.block_diag_rotate(kh, d.had_block)
        errs[rot] = float(np.linalg.norm(kh - k_rope) / np.linalg.norm(k_rope))
    say("relative key error without / with rotation", errs[False], errs[True])
    assert errs[True] < 0.5 * errs[False], errs


# ---------------------------------------------------------------- projections


def _check_int4_linear(F, DB, shape, d, proj, m, g, batch, r):
    n, kk = m.shape
    act = W.to_bf16_values(r.standard_normal((batch, kk)).astype(np.float32))
    abits = (act.view(np.uint32) >> 16).astype(np.uint16)
    pp = DB.pack_projection(d, proj, m, g)
    ws_bytes = F.futx_decode_workspace_size(d, batch, 1)
    ws = DB.device_buffer(ws_bytes)
    out = torch.empty((batch, n), dtype=torch.float32, device="cuda")
    say("int4_linear", shape, proj, "batch", batch)
    F.futx_int4_linear(d, proj, (pp.packed, pp.scales), batch, torch.from_numpy(abits).cuda(), out, ws,
                       ws_bytes)
    torch.cuda.synchronize()
    folded = m if g is None else oracle.fold_gain(m, g)
    q, s = oracle.quantize_weight_rtn(folded, d.w_group)
    ref = act.astype(np.float64) @ oracle.dequant_weight(q, s, d.w_group).T
    err = np.max(np.abs(out.cpu().numpy() - ref))
    say("  max err %.3g  (max|ref| %.3g)" % (err, np.max(np.abs(ref))))
    # fp32 accumulation over K inputs: far below the block tolerance
    assert err <= 1e-5 * np.max(np.abs(ref)) * np.sqrt(kk / 128) + 1e-6, (proj, err)


@pytest.mark.parametrize("shape", ["tiny", "8b"])
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 16, 17, 32])
def test_int4_linear(F, DB, shape, batch):
    # batches 1-5 cross the planner's workgroup shapes: 4-wave workgroups, and
    # 16-wave ones for the large projections from batch 2 and all from batch 4
    wl = W.tiny() if shape == "tiny" else W.llama8b()
    w = W.block_weights(wl, 0)
    r = np.random.default_rng(23 + batch)
    for proj, m, g in (("qkv", w["wqkv"], w["gain_attn"]), ("o", w["wo"], None),
                       ("gateup", np.concatenate([w["wgate"], w["wup"]]), w["gain_ffn"]), ("down", w["wdown"], None)):
        if shape == "8b" and proj in ("qkv", "o") and batch not in (1, 2, 4, 32):
            continue
        _check_int4_linear(F, DB, shape, wl.dims, proj, m, g, batch, r)


@pytest.mark.slow
@pytest.mark.parametrize("batch", [2, 3])
def test_int4_linear_70b(F, DB, batch):
    """Llama-3-70B-shape QKV, O and down projections at batches 2 and 3, where
    they take 16-wave workgroups (down at batch 3 as a K split with its
    finishing kernel)."""
    d = W.llama70b(batch).dims
    r = np.random.default_rng(31 + batch)
    nq_d = d.n_heads * d.head_dim
    for proj, shape, gained in (("qkv", (d.n_qkv, d.hidden), True), ("o", (d.hidden, nq_d), False),
                                ("down", (d.hidden, d.intermediate), False)):
        m = (r.standard_normal(shape) * 0.02).astype(np.float32)
        g = r.uniform(0.5, 1.5, d.hidden).astype(np.float32) if gained else None
        _check_int4_linear(F, DB, "70b", d, proj, m, g, batch, r)


def test_int4_linear_external_codes(F, DB):
    """Weights that enter as external codes and scales (full code range,
    -8 included) through futx_pack_codes: the projection equals the fp64
    product with the dequantized weights."""
    d = W.LLAMA8B
    r = np.random.default_rng(41)
    for proj, (n, kk) in (("o", (4096, 4096)), ("down", (4096, 14336))):
        q = r.integers(-8, 8, (n, kk)).astype(np.int8)
        s = (np.abs(r.standard_normal((n, kk // d.w_group))) * 0.003).astype(np.float16)
        pb, sb = F.futx_packed_sizes(d, proj)
        packed, scales = DB.device_buffer(pb), DB.device_buffer(sb)
        F.futx_pack_codes(d, proj, oracle.pack_nibbles(q), s.view(np.uint16), packed, scales)
        for batch in (1, 8):
            act = W.to_bf16_values(r.standard_normal((batch, kk)).astype(np.float32))
            abits = (act.view(np.uint32) >> 16).astype(np.uint16)
            ws_bytes = F.futx_decode_workspace_size(d, batch, 1)
            ws = DB.device_buffer(ws_bytes)
            out = torch.empty((batch, n), dtype=torch.float32, device="cuda")
            say("int4_linear external codes", proj, "batch", batch)
            F.futx_int4_linear(d, proj, (packed, scales), batch, torch.from_numpy(abits).cuda(), out, ws, ws_bytes)
            torch.cuda.synchronize()
            ref = act.astype(np.float64) @ oracle.dequant_weight(q, s, d.w_group).T
            err = np.max(np.abs(out.cpu().numpy() - ref))
            say("  max err %.3g  (max|ref| %.3g)" % (err, np.max(np.abs(ref))))
            assert err <= 1e-5 * np.max(np.abs(ref)) * np.sqrt(kk / 128) + 1e-6, (proj, batch, err)


# ---------------------------------------------------------------- attention


ATTN_SHAPES = {"tiny": W.TINY, "8b": W.LLAMA8B, "70b": W.LLAMA70B}


def _attention_case(DB, shape, lens, max_context=None, seed=24):
    """Device cache with `lens[b]` cached tokens per sequence (quantizer only,
    from rotated fp32 values, so device and oracle hold the same codes), a
    random fp32 QKV projection, and futx_decode_attention (the attention
    stage of the block: append of the new token at cached_lens[b], queries,
    splits, merge, inverse rotation).  Returns (out, oracle pieces)."""
    d = ATTN_SHAPES[shape]
    wl = W.Workload(f"attn-{shape}", d, len(lens), "fixed:0")
    lens = np.asarray(lens, np.int32)
    mc = int(max_context) if max_context else int(lens.max()) + 1
    layout = W.page_layout(wl, np.minimum(lens, mc - 1), extra_tokens=1, seed=5, spare_pages=2)
    r = np.random.default_rng(seed)
    cache = DB.DeviceKVCache(d, layout.num_pages)
    hist = []
    for b, L in enumerate(lens):
        L = min(int(L), mc - 1)
        kr = r.standard_normal((L, d.n_kv_heads, d.head_dim)).astype(np.float32)
        vr = (r.standard_normal((L, d.n_kv_heads, d.head_dim)) * 2).astype(np.float32)
        if L:
            slots = (layout.block_table[b, np.arange(L) // 64] * 64 + np.arange(L) % 64).astype(np.int32)
            cache.append(torch.from_numpy(kr).cuda(), torch.from_numpy(vr).cuda(), None,
                         torch.from_numpy(slots).cuda(), flags=0)
        hist.append((kr, vr))
    qkv = r.standard_normal((len(lens), d.n_qkv)).astype(np.float32)
    qkv[:, : d.n_heads * d.head_dim] *= 2
    return d, lens, mc, layout, cache, hist, qkv


def _run_attention(F, DB, d, lens, mc, layout, cache, qkv, reps=1):
    ws_bytes = F.futx_decode_workspace_size(d, len(lens), mc)
    ws = DB.device_buffer(ws_bytes)
    outs = []
    for _ in range(reps):
        out = torch.empty((len(lens), d.n_heads, d.head_dim), dtype=torch.float32, device="cuda")
        F.futx_decode_attention(d, len(lens), torch.from_numpy(qkv).cuda(), torch.from_numpy(lens).cuda(),
                                torch.from_numpy(layout.block_table).cuda(), layout.block_table.shape[1], mc,
                                cache.c_cache, out, ws, ws_bytes)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    return outs


def _oracle_attention(d, b, L, hist, qkv, K, KS, V, VS, flips):
    """Oracle attention of sequence b: history codes from the oracle's
    quantizer (the same codes as the device's), the new token from the
    oracle's RoPE + rotation, with its boundary decisions checked against the
    device's codes (flip_tolerant) and then taken from them."""
    nq, nkv, D = d.n_heads, d.n_kv_heads, d.head_dim
    kr, vr = hist[b]
    c = oracle.LogicalKVCache.empty(L + 1, nkv, D)
    if L:
        c.k_codes[:L], c.k_scales[:L] = oracle.quantize_kv_token(kr)
        c.v_codes[:L], c.v_scales[:L] = oracle.quantize_kv_token(vr)
    row = qkv[b].astype(np.float64)
    q = row[: nq * D].reshape(nq, D)
    k = row[nq * D:(nq + nkv) * D].reshape(nkv, D)
    v = row[(nq + nkv) * D:].reshape(nkv, D)
    q_rot = oracle.block_diag_rotate(oracle.rope_rotate_half(q, L, d.rope_theta), d.had_block)
    k_rot, v_rot = oracle.rotate_kv(k, v, L, d)
    flips.add(flip_tolerant(K[b], KS[b], k_rot, ("attention new key", b), max_frac=1.0, max_per_row=1))
    flips.add(flip_tolerant(V[b], VS[b], v_rot, ("attention new value", b), max_frac=1.0, max_per_row=1))
    c.write(L, K[b], KS[b], V[b], VS[b])
    k_hat, v_hat = c.dequant(L + 1)
    return oracle.decode_attention(q_rot, k_hat, v_hat, d.had_block)


# accuracy of the attention output: the O projection takes it as two bf16
# terms (relative error 2^-18), so the kernel itself must be at least that
# accurate for that operand to add no rounding point of its own
ATTN_RTOL = 2.0 ** -18


RAGGED_32 = [int(v) for v in W.llama8b_ragged(32).cached_lengths(0)]


@pytest.mark.parametrize("shape,lens", [("tiny", [0]), ("tiny", [63, 64, 65, 200]), ("8b", [2048]),
                                        ("8b", [0, 31, 32, 33, 700, 4096]), ("70b", [129, 1000]),
                                        ("8b", RAGGED_32)])
def test_decode_attention(F, DB, shape, lens):
    """The hot-path attention kernel through futx_decode_attention: every
    output element within 2^-18 max|o| of the fp64 oracle."""
    d, lens, mc, layout, cache, hist, qkv = _attention_case(DB, shape, lens)
    say("decode_attention", shape, lens.tolist())
    got = _run_attention(F, DB, d, lens, mc, layout, cache, qkv)[0]
    slots = np.array([layout.slot(b, int(L)) for b, L in enumerate(lens)], np.int32)
    K, KS, V, VS = _cache_tokens(cache.host_copy(), d, layout.num_pages, slots)
    flips = FlipStats()
    for b, L in enumerate(lens):
        ref = _oracle_attention(d, b, int(L), hist, qkv, K, KS, V, VS, flips)
        err = float(np.max(np.abs(got[b] - ref)))
        tol = ATTN_RTOL * float(np.max(np.abs(ref))) + 1e-7
        say("  b", b, "L", int(L), "max err %.3g (%.2e of max|o|) tol %.3g" % (err, err / np.max(np.abs(ref)), tol))
        assert err <= tol, (b, err, tol)
    say("  new token:", flips)


@pytest.mark.parametrize("shape,batch,length", [("8b", 32, 4096), ("70b", 8, 4096), ("8b", 1, 2048)])
def test_decode_attention_repeatable(F, DB, shape, batch, length):
    """Large shapes (several workgroups per sequence, merged by the last to
    arrive): three runs give bit-identical outputs whatever the arrival
    order, and sampled rows match the oracle."""
    d, lens, mc, layout, cache, hist, qkv = _attention_case(DB, shape, [length] * batch, seed=25)
    say("decode_attention repeatability", shape, "batch", batch, "L", length)
    outs = _run_attention(F, DB, d, lens, mc, layout, cache, qkv, reps=3)
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])
    slots = np.array([layout.slot(b, int(L)) for b, L in enumerate(lens)], np.int32)
    K, KS, V, VS = _cache_tokens(cache.host_copy(), d, layout.num_pages, slots)
    flips = FlipStats()
    for b in sorted({0, batch // 2, batch - 1}):
        ref = _oracle_attention(d, b, int(lens[b]), hist, qkv, K, KS, V, VS, flips)
        err = float(np.max(np.abs(outs[0][b] - ref)))
        tol = ATTN_RTOL * float(np.max(np.abs(ref))) + 1e-7
        say("  b", b, "max err %.3g tol %.3g" % (err, tol))
        assert err <= tol, (b, err, tol)


def test_decode_attention_length_outside_plan(F, DB):
    """A cached length with cached_lens[b] + 1 > max_context: that sequence's
    output is NaN and its cache slot is not written; the other sequences are
    unaffected."""
    d, lens, mc, layout, cache, hist, qkv = _attention_case(DB, "tiny", [100, 300, 64], max_context=257)
    assert lens[1] + 1 > mc
    before = cache.host_copy()
    say("decode_attention with a length outside the plan", lens.tolist(), "max_context", mc)
    got = _run_attention(F, DB, d, lens, mc, layout, cache, qkv)[0]
    assert np.all(np.isnan(got[1]))
    assert not np.any(np.isnan(got[[0, 2]]))
    slots = np.array([layout.slot(b, int(min(L, mc - 1))) for b, L in enumerate(lens)], np.int32)
    K0, KS0, V0, VS0 = _cache_tokens(before, d, layout.num_pages, slots)
    K, KS, V, VS = _cache_tokens(cache.host_copy(), d, layout.num_pages, slots)
    np.testing.assert_array_equal(K[1], K0[1])
    np.testing.assert_array_equal(V[1], V0[1])
    flips = FlipStats()
    for b in (0, 2):
        ref = _oracle_attention(d, b, int(lens[b]), hist, qkv, K, KS, V, VS, flips)
        assert float(np.max(np.abs(got[b] - ref))) <= ATTN_RTOL * float(np.max(np.abs(ref))) + 1e-7


# ---------------------------------------------------------------- whole block


def _check_block(case, reps=2):
    outs = case.run_gpu(reps=reps)
    y = case.run_oracle()
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])  # deterministic: bitwise repeatable
    err = float(np.max(np.abs(outs[0] - y)))
    tol = block_tolerance(y)
    if err > tol:
        rows = np.max(np.abs(outs[0] - y), axis=1) / tol
        say(case.wl.name, "per-row err / tol", np.round(rows, 3).tolist(), "lens", case.lens.tolist())
    say(case.wl.name, "block max err %.4g tol %.4g (%.3f of tol); %d runs bitwise equal; history: %s; new token: %s"
        % (err, tol, err / tol, reps, case.hist_flips, case.kv_flips))
    assert err <= tol, (case.wl.name, err, tol, str(case.hist_flips), str(case.kv_flips))
    return outs[0], y


def test_block_tiny():
    case = BlockCase(W.tiny())
    _check_block(case)
    # the new token sits in the cache at position cached_lens: the oracle's
    # kv_hook read it from that slot and checked it against the oracle's own
    # quantization (differences only at rounding boundaries)
    assert case.kv_flips is not None
    d = case.dims
    L = int(case.lens[0])
    slot = np.array([case.layout.slot(0, L)], np.int32)
    K, KS, V, VS = _cache_tokens(case.gpu_cache, d, case.layout.num_pages, slot)
    oc = case.oracle_caches[0]
    np.testing.assert_array_equal(K[0], oc.k_codes[L])
    np.testing.assert_array_equal(V[0], oc.v_codes[L])


@pytest.mark.parametrize("batch,lens", [(3, "fixed:0"), (4, "uniform:1:200"), (17, "uniform:1:200")])
def test_block_tiny_ragged(batch, lens):
    # batch 17: the projections run in batch tiles of unequal row counts
    wl = W.Workload(f"tiny-ragged-b{batch}-{lens}", W.TINY, batch, lens)
    _check_block(BlockCase(wl))


def test_block_8b():
    _check_block(BlockCase(W.llama8b()), reps=1)


@pytest.mark.parametrize("batch", [1, 4, 8, 16, 17, 32])
def test_block_8b_ragged_outliers(batch):
    # batches 16, 17 and 32 run the projections in batch tiles (17: tiles of
    # unequal row counts)
    # batch 32 (split-K projections and their reduce kernels) runs twice and
    # must repeat bit for bit
    _check_block(BlockCase(W.llama8b_ragged(batch)), reps=2 if batch == 32 else 1)


@pytest.mark.parametrize("shape,x_scale", [("tiny", 8.0), ("tiny", 1.0 / 16), ("8b", 8.0), ("8b", 1.0 / 16)])
def test_block_input_far_from_unit_rms(shape, x_scale):
    """Block inputs with RMS 8 and 1/16 instead of about 1: the RMSNorm scale
    1/r enters the QKV and gate/up epilogues, so a misapplied scale shows up
    here even where unit-RMS inputs would hide it."""
    wl = W.tiny(2) if shape == "tiny" else W.llama8b(1)
    _check_block(BlockCase(wl, x_scale=x_scale), reps=1)


@pytest.mark.slow
@pytest.mark.parametrize("batch", [1, 4, 8, 16, 32])
def test_block_70b(batch):
    """Llama-3-70B-shape block (hidden 8192, 64/8 heads, intermediate 28672),
    4096 cached tokens per sequence."""
    _check_block(BlockCase(W.llama70b(batch)), reps=2 if batch == 8 else 1)


@pytest.mark.parametrize("shape,lens", [("tiny", [61, 0, 127]), ("8b", [62, 300])])
def test_multi_step_decode(F, DB, shape, lens):
    """Several decode steps in a row on one cache: each step appends its new
    token at slot cached_lens[b] (crossing page boundaries into pages drawn
    from a seeded permutation), the caller then advances cached_lens, and
    the next step attends to every token written so far.  Each step's output
    is checked against the oracle block continuing on its own cache (the
    new token's boundary-case codes taken from the device, as in the
    single-block tests)."""
    from tests.gpu_common import cache_tokens

    steps = 4
    dims = W.TINY if shape == "tiny" else W.LLAMA8B
    wl = W.Workload(f"multistep-{shape}", dims, len(lens), "fixed:0")
    d = wl.dims
    lens = np.asarray(lens, np.int32)
    layout = W.page_layout(wl, lens, extra_tokens=steps, seed=0, spare_pages=1)
    w = W.block_weights(wl, 0)
    hist = [W.history(wl, 0, b, int(L)) for b, L in enumerate(lens)]
    layer = DB.DeviceLayer(d, w)
    cache = DB.DeviceKVCache(d, layout.num_pages)
    for b, (k, v) in enumerate(hist):
        DB.fill_history(cache, k, v, layout, b)
    qw = oracle.quantize_block_weights(w, d)
    torch.cuda.synchronize()
    dec = DecodedCache(cache.host_copy(), d, layout.num_pages)
    hist_flips = FlipStats()
    ocaches = [oracle_history(dec, d, layout, b, k, v, int(lens[b]) + steps, hist_flips)
               for b, (k, v) in enumerate(hist)]
    say("multi-step decode", shape, "history:", hist_flips)
    for t in range(steps):
        cur = lens + t
        x = W.hidden_state(wl, tag=f"x{t}")
        runner = DB.DecodeRunner(d, wl.batch, cur, layout.block_table)
        xd = torch.from_numpy(x.copy()).cuda()
        say("multi-step decode", shape, "step", t, "cached_lens", cur.tolist())
        runner.decode(layer, cache, xd)
        torch.cuda.synchronize()
        got = xd.cpu().numpy()
        slots = np.array([layout.slot(b, int(L)) for b, L in enumerate(cur)], np.int32)
        K, KS, V, VS = cache_tokens(cache.host_copy(), d, layout.num_pages, slots)

        flips = FlipStats()

        def hook(b, kc, ks, vc, vs, k_rot, v_rot):
            flips.add(_flip_tolerant(K[b], KS[b], np.asarray(k_rot, np.float64), ("new key", t, b), max_frac=1.0,
                                     max_per_row=1))
            flips.add(_flip_tolerant(V[b], VS[b], np.asarray(v_rot, np.float64), ("new value", t, b), max_frac=1.0,
                                     max_per_row=1))
            return K[b].astype(kc.dtype), KS[b].astype(ks.dtype), V[b].astype(vc.dtype), VS[b].astype(vs.dtype)

        ref = oracle.decode_block(x, qw, ocaches, cur, d, kv_hook=hook)
        err = float(np.max(np.abs(got - ref)))
        tol = block_tolerance(ref)
        say("  step %d max err %.3g tol %.3g; new token: %s" % (t, err, tol, flips))
        assert err <= tol, (t, err, tol)
