"""GPU parity of a generation loop (int4_weight_kv_amd.block.DecodeSession):
unpadded prompts placed through futx_kv_append, then T decode steps in which
each step's top-1 token is the next step's input (fed back on the device
through futx_embed), cache pages are taken from a seeded free list as
sequences cross page boundaries, and every step is checked against the
oracle layer by layer (each block on the step's own input, the history and
new-token codes continuing with the device's choice where they sit on a
rounding boundary), and the LM head on the step's final state."""

import numpy as np
import pytest

import oracle
from int4_weight_kv_amd import workload as W

from .gpu_common import DecodedCache, FlipStats, block_tolerance, flip_tolerant, oracle_history, say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def DB():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from int4_weight_kv_amd import block

    return block


@pytest.mark.parametrize("shape,prompts,steps", [("tiny", [61, 0, 127], 6), ("8b", [62, 190], 4)])
def test_generation_loop(DB, shape, prompts, steps):
    dims = W.TINY if shape == "tiny" else W.LLAMA8B
    n_layers = 3 if shape == "tiny" else 2
    batch = len(prompts)
    wl = W.Workload(f"gen-{shape}", dims, batch, "fixed:0", n_layers=n_layers, vocab=512)
    d = dims
    prompts = np.asarray(prompts, np.int32)
    max_context = int(prompts.max()) + steps + 1
    ws = [W.block_weights(wl, li) for li in range(n_layers)]
    layers = [DB.DeviceLayer(d, w) for w in ws]
    qws = [oracle.quantize_block_weights(w, d) for w in ws]
    del ws
    emb, head, gain = W.lm_tables(wl)
    dh = DB.DecodeHead(d, emb, head, gain, batch)
    folded = oracle.fold_head(head, gain)
    num_pages = int(sum((p + steps + 63) // 64 for p in prompts)) + 2
    sess = DB.DecodeSession(d, layers, dh, batch, num_pages, max_context, page_seed=11)
    hist = {}
    for b, L in enumerate(prompts):
        kv = [W.history(wl, li, b, int(L)) for li in range(n_layers)]
        hist[b] = kv
        sess.place_prompt(b, [k for k, _ in kv], [v for _, v in kv])
    torch.cuda.synchronize()
    say("generation", shape, "prompts", prompts.tolist(), "pages after prompts",
        [int((sess.paged.table[b] >= 0).sum()) for b in range(batch)])

    # the oracle's caches: the prompts as the device wrote them (boundary cases checked)
    flips_hist = FlipStats()
    ocaches = []
    for li in range(n_layers):
        dec = DecodedCache(sess.caches[li].host_copy(), d, num_pages)
        layout = W.PageLayout(sess.paged.table.copy(), num_pages)
        ocaches.append([oracle_history(dec, d, layout, b, hist[b][li][0], hist[b][li][1], int(prompts[b]) + steps,
                                       flips_hist) for b in range(batch)])
    say("  prompt boundary decisions taken from the device:", flips_hist)

    tokens = torch.from_numpy(W.tokens(wl)).cuda()
    flips_new = FlipStats()
    worst = 0.0
    for t in range(steps):
        lens_t = sess.paged.lens.copy()
        pages_before = (sess.paged.table >= 0).sum(axis=1)
        tok_host = tokens.cpu().numpy().copy()
        xs = []

        def grab(i, x):
            torch.cuda.synchronize()
            xs.append(x.cpu().numpy().copy())

        x_in = None
        top1 = sess.step(tokens, progress=grab)
        torch.cuda.synchronize()
        # pages: one taken exactly where the new token starts a page
        pages_after = (sess.paged.table >= 0).sum(axis=1)
        want = ((lens_t % 64 == 0) & (lens_t // 64 >= pages_before)).astype(int)
        assert list(pages_after - pages_before) == list(want), (t, lens_t.tolist())
        used = sess.paged.table[sess.paged.table >= 0]
        assert len(set(used.tolist())) == len(used)
        # the block inputs: the embedding of this step's tokens, exactly
        x0 = np.asarray(emb, np.float32)[tok_host]
        ins = [x0] + xs[:-1]
        layout = W.PageLayout(sess.paged.table.copy(), num_pages)
        slots = np.array([layout.slot(b, int(L)) for b, L in enumerate(lens_t)], np.int32)
        for li in range(n_layers):
            dec = DecodedCache(sess.caches[li].host_copy(), d, num_pages)
            K, KS, V, VS = dec.tokens(slots)

            def hook(b, kc, ks, vc, vs, k_rot, v_rot):
                flips_new.add(flip_tolerant(K[b], KS[b], np.asarray(k_rot, np.float64), ("new key", t, li, b),
                                            max_frac=1.0, max_per_row=1))
                flips_new.add(flip_tolerant(V[b], VS[b], np.asarray(v_rot, np.float64), ("new value", t, li, b),
                                            max_frac=1.0, max_per_row=1))
                return K[b].astype(kc.dtype), KS[b].astype(ks.dtype), V[b].astype(vc.dtype), VS[b].astype(vs.dtype)

            ref = oracle.decode_block(ins[li], qws[li], ocaches[li], lens_t, d, kv_hook=hook)
            err = float(np.max(np.abs(xs[li] - ref)))
            tol = block_tolerance(ref)
            worst = max(worst, err / tol)
            assert err <= tol, (t, li, err, tol)
        # the LM head on the step's final state, and the top-1 rule
        ref_logits, ref_top1 = oracle.lm_head(xs[-1], folded, d.rms_eps)
        got_logits = sess.logits.cpu().numpy()
        got_top1 = top1.cpu().numpy()
        ltol = block_tolerance(ref_logits)
        lerr = float(np.max(np.abs(got_logits - ref_logits)))
        assert lerr <= ltol, (t, lerr, ltol)
        for b in range(batch):
            if got_top1[b] != ref_top1[b]:
                gap = ref_logits[b, ref_top1[b]] - ref_logits[b, got_top1[b]]
                assert gap <= ltol, (t, b, gap, ltol)
        say("  step", t, "lens", lens_t.tolist(), "tokens in", tok_host.tolist(), "top-1", got_top1.tolist(),
            "pages", pages_after.tolist(), "logits err %.3g tol %.3g" % (lerr, ltol))
        # the next step's input is this step's top-1, on the device
        tokens = top1
    say("  worst block err / tol %.3f; new-token boundary decisions taken from the device: %s" % (worst, flips_new))
    np.testing.assert_array_equal(sess.paged.lens, prompts + steps)
