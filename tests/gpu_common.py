"""Shared set-up of the GPU parity tests: one decode-block case built twice,
once on the device through the C ABI and once in the CPU oracle, from the
same seeded inputs (int4_weight_kv_amd.workload)."""

import sys
import time

import numpy as np

import oracle
from int4_weight_kv_amd import workload as W


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def flip_tolerant(got_q, got_s, x64, tag, max_frac=1e-4):
    """Compare implementation codes/scales with the oracle's fp32 recipe
    applied to the oracle's fp64 values.  Allowed differences (fp32 on the GPU
    vs fp64 in the oracle before the fp32 quantizer):
      * a scale one fp16 step away, only where the oracle's fp32(max/7) lies
        within 2**-20 (relative) of the midpoint of the two fp16 values;
      * a code one step away, only where the oracle's value / scale lies
        within 1e-3 of a half-integer (1e-2 on rows whose scale moved), and on
        at most `max_frac` of the elements.
    Returns (code flips, scale flips)."""
    x32 = x64.astype(np.float32)
    want_q, want_s = oracle.quantize_kv_token(x32)
    s_bad = got_s.view(np.uint16) != want_s.view(np.uint16)
    if np.any(s_bad):
        step = np.abs(got_s.view(np.uint16)[s_bad].astype(np.int64) - want_s.view(np.uint16)[s_bad].astype(np.int64))
        assert np.all(step == 1), tag
        s32 = (np.max(np.abs(x32), axis=-1) / np.float32(7)).astype(np.float32)[s_bad].astype(np.float64)
        mid = (got_s[s_bad].astype(np.float64) + want_s[s_bad].astype(np.float64)) / 2
        assert np.all(np.abs(s32 - mid) <= 2.0 ** -20 * s32), (tag, s32, mid)
    q_bad = got_q != want_q
    if np.any(q_bad):
        assert np.all(np.abs(got_q.astype(np.int16) - want_q)[q_bad] <= 1), tag
        sf = want_s.astype(np.float64)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            r = x64 / sf
        frac = np.abs(r - np.floor(r) - 0.5)
        lim = np.where(np.broadcast_to(s_bad[..., None], q_bad.shape), 1e-2, 1e-3)
        assert np.all(frac[q_bad] < lim[q_bad]), tag
    assert q_bad.mean() <= max_frac, (tag, q_bad.mean())
    return int(q_bad.sum()), int(s_bad.sum())


def cache_tokens(cache_host, dims, num_pages, slots):
    """Codes and scales of the given cache slots: K [n][nkv][d], KS [n][nkv], V, VS."""
    from . import layouts

    kc, vc, ks, vs = cache_host
    K, KS, V, VS = layouts.decode_cache(kc, vc, ks, vs, num_pages, dims.n_kv_heads, dims.head_dim)
    p, o = np.asarray(slots) // 64, np.asarray(slots) % 64
    return K[p, :, o], KS[p, :, o], V[p, :, o], VS[p, :, o]


def block_tolerance(ref):
    """Acceptance bound of a block output: 2e-3 * max|oracle| + 1e-3."""
    return 2e-3 * float(np.max(np.abs(ref))) + 1e-3


class BlockCase:
    """Inputs of one decode-block workload (host, numpy)."""

    def __init__(self, wl: W.Workload, seed=0, layer=0, spare_pages=3):
        self.wl, self.seed, self.layer = wl, seed, layer
        self.dims = wl.dims
        self.lens = wl.cached_lengths(seed)
        self.layout = W.page_layout(wl, self.lens, extra_tokens=1, seed=seed, spare_pages=spare_pages)
        self.w = W.block_weights(wl, layer, seed)
        self.x = W.hidden_state(wl, seed)
        self.hist = [W.history(wl, layer, b, int(L), seed) for b, L in enumerate(self.lens)]

    # ---------------------------------------------------------------- device
    def run_gpu(self, reps=1):
        import torch

        from int4_weight_kv_amd import block as DB

        d = self.dims
        say("device set-up", self.wl.name, "lens", self.lens.tolist()[:8])
        layer = DB.DeviceLayer(d, self.w)
        cache = DB.DeviceKVCache(d, self.layout.num_pages)
        for b, (k, v) in enumerate(self.hist):
            DB.fill_history(cache, k, v, self.layout, b)
        runner = DB.DecodeRunner(d, self.wl.batch, self.lens, self.layout.block_table)
        outs = []
        for _ in range(reps):
            xd = torch.from_numpy(self.x.copy()).cuda()
            say("futx_decode_block", self.wl.name, "batch", self.wl.batch)
            runner.decode(layer, cache, xd)
            torch.cuda.synchronize()
            outs.append(xd.cpu().numpy())
        self.gpu_cache = cache.host_copy()
        return outs

    # ---------------------------------------------------------------- oracle
    def gpu_kv_hook(self):
        """kv_hook for oracle.decode_block: the new token's codes and scales as
        the GPU wrote them, after checking that every difference from the
        oracle's own quantization is a rounding-boundary case."""
        d = self.dims
        slots = np.array([self.layout.slot(b, int(L)) for b, L in enumerate(self.lens)], np.int32)
        K, KS, V, VS = cache_tokens(self.gpu_cache, d, self.layout.num_pages, slots)
        self.kv_flips = [0, 0]

        def hook(b, kc, ks, vc, vs, k_rot, v_rot):
            fk = flip_tolerant(K[b], KS[b], np.asarray(k_rot, np.float64), ("new key", b), max_frac=1.0)
            fv = flip_tolerant(V[b], VS[b], np.asarray(v_rot, np.float64), ("new value", b), max_frac=1.0)
            self.kv_flips[0] += fk[0] + fv[0]
            self.kv_flips[1] += fk[1] + fv[1]
            return K[b].astype(kc.dtype), KS[b].astype(ks.dtype), V[b].astype(vc.dtype), VS[b].astype(vs.dtype)

        return hook

    def run_oracle(self, gpu_codes=True):
        """The oracle block; with gpu_codes (after run_gpu), the new token's
        boundary-case codes follow the GPU's choice (gpu_kv_hook)."""
        d = self.dims
        t0 = time.time()
        qw = oracle.quantize_block_weights(self.w, d)
        caches = []
        for b, (k, v) in enumerate(self.hist):
            L = int(self.lens[b])
            c = oracle.LogicalKVCache.empty(L + 1, d.n_kv_heads, d.head_dim)
            if L:
                oracle.history_fill(c, k, v, np.arange(L), d)
            caches.append(c)
        diag = {}
        hook = self.gpu_kv_hook() if gpu_codes and getattr(self, "gpu_cache", None) is not None else None
        y = oracle.decode_block(self.x, qw, caches, self.lens, d, diag=diag, kv_hook=hook)
        if hook is not None and sum(self.kv_flips):
            say("new-token boundary flips taken from the GPU (codes, scales):", self.kv_flips)
        self.oracle_caches, self.diag = caches, diag
        say("oracle done in %.1fs" % (time.time() - t0))
        return y
