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


# Code-boundary window, in code units (value / scale).  The device forms the
# new token's key and value in fp32: an fp32-accumulated INT4 projection
# (relative error about 1e-6), the 1/r scale, RoPE with fp32 cos / sin and the
# Hadamard butterflies (a few fp32 roundings each); value / scale is at most
# 7.5, so the device's value / scale differs from the fp64 one by about 1e-5.
# A code may differ from the oracle's only where the oracle's value / scale
# lies within ten times that of a rounding midpoint.
CODE_WINDOW = 1e-4
# fp16 scale-boundary window (relative to fp32(max / 7)), from the same error
SCALE_WINDOW = 2.0 ** -20


class FlipStats:
    """Boundary decisions where an implementation and the oracle differ."""

    def __init__(self):
        self.codes = 0
        self.scales = 0
        self.rows = 0
        self.worst = 0.0  # largest |value / scale - midpoint| among code flips

    def add(self, other):
        self.codes += other.codes
        self.scales += other.scales
        self.rows += other.rows
        self.worst = max(self.worst, other.worst)

    def __repr__(self):
        return (f"{self.codes} code flips, {self.scales} scale flips over {self.rows} rows "
                f"(farthest {self.worst:.2e} from a midpoint; window {CODE_WINDOW:g})")


def flip_tolerant(got_q, got_s, x64, tag, max_frac=1e-4, max_per_row=None):
    """Compare implementation codes/scales [..., d] / [...] with the oracle's
    fp32 recipe applied to the oracle's fp64 values x64.  Allowed differences:
      * a scale one fp16 step away, only where the oracle's fp32(max/7) lies
        within SCALE_WINDOW (relative) of the midpoint of the two fp16 values;
      * a code one step away from the recipe applied with the scale the
        implementation stored, only where the oracle's value / that scale lies
        within CODE_WINDOW of a half-integer;
      * at most `max_frac` of the elements, and at most `max_per_row` flipped
        codes in any one row (None: no per-row cap).
    Returns FlipStats."""
    st = FlipStats()
    st.rows = int(np.prod(got_s.shape))
    x32 = x64.astype(np.float32)
    want_q, want_s = oracle.quantize_kv_token(x32)
    s_bad = got_s.view(np.uint16) != want_s.view(np.uint16)
    if np.any(s_bad):
        step = np.abs(got_s.view(np.uint16)[s_bad].astype(np.int64) - want_s.view(np.uint16)[s_bad].astype(np.int64))
        assert np.all(step == 1), (tag, "scale more than one fp16 step away")
        s32 = (np.max(np.abs(x32), axis=-1) / np.float32(7)).astype(np.float32)[s_bad].astype(np.float64)
        mid = (got_s[s_bad].astype(np.float64) + want_s[s_bad].astype(np.float64)) / 2
        assert np.all(np.abs(s32 - mid) <= SCALE_WINDOW * s32), (tag, s32, mid)
        st.scales = int(s_bad.sum())
    # the recipe with the stored scale (equal to the oracle's except on the
    # rows checked above)
    s_used = got_s.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        exp_q = np.where(s_used == 0, np.float32(0), np.clip(np.rint((x32 / s_used).astype(np.float32)), -8, 7))
    exp_q = exp_q.astype(np.int8)
    q_bad = got_q != exp_q
    if np.any(q_bad):
        assert np.all(np.abs(got_q.astype(np.int16) - exp_q)[q_bad] <= 1), (tag, "code more than one step away")
        with np.errstate(divide="ignore", invalid="ignore"):
            r = x64 / s_used.astype(np.float64)
        dist = np.abs(r - np.floor(r) - 0.5)
        assert np.all(dist[q_bad] < CODE_WINDOW), (tag, "code flip away from a midpoint", float(dist[q_bad].max()))
        st.codes = int(q_bad.sum())
        st.worst = float(dist[q_bad].max())
        if max_per_row is not None:
            per_row = q_bad.reshape(-1, q_bad.shape[-1]).sum(axis=1)
            assert per_row.max() <= max_per_row, (tag, "flips in one row", int(per_row.max()))
    assert q_bad.mean() <= max_frac, (tag, q_bad.mean())
    return st


class DecodedCache:
    """A host copy of a device KV cache decoded once (tests/layouts.py):
    codes K, V [page][nkv][64][d] and scales KS, VS [page][nkv][64]."""

    def __init__(self, cache_host, dims, num_pages):
        from . import layouts

        kc, vc, ks, vs = cache_host
        self.K, self.KS, self.V, self.VS = layouts.decode_cache(kc, vc, ks, vs, num_pages, dims.n_kv_heads,
                                                                dims.head_dim)

    def tokens(self, slots):
        p, o = np.asarray(slots) // 64, np.asarray(slots) % 64
        return self.K[p, :, o], self.KS[p, :, o], self.V[p, :, o], self.VS[p, :, o]


def cache_tokens(cache_host, dims, num_pages, slots):
    """Codes and scales of the given cache slots: K [n][nkv][d], KS [n][nkv], V, VS."""
    dec = cache_host if isinstance(cache_host, DecodedCache) else DecodedCache(cache_host, dims, num_pages)
    return dec.tokens(slots)


def oracle_history(decoded, dims, layout, b, k, v, cap, stats):
    """The oracle's cache of sequence b with len(k) history tokens at
    positions 0.. (pre-RoPE fp32 k, v [L][nkv][d]) and room for `cap` tokens.
    The oracle rotates them in fp64 (RoPE, block Hadamard) and quantizes them
    by its fp32 recipe; where the device, which rotated them in fp32, stored a
    code or scale on the other side of a rounding boundary (flip_tolerant: at
    most one code per token and head, within CODE_WINDOW of a midpoint), the
    oracle continues with the device's choice, as it does for the new token.
    decoded: the device cache (DecodedCache), or None for the oracle's own
    codes throughout."""
    L = len(k)
    c = oracle.LogicalKVCache.empty(cap, dims.n_kv_heads, dims.head_dim)
    if L == 0:
        return c
    pos = np.arange(L)
    if decoded is None:
        oracle.history_fill(c, k, v, pos, dims)
        return c
    k_rot, v_rot = oracle.rotate_kv(np.asarray(k, np.float64), np.asarray(v, np.float64), pos[:, None], dims)
    slots = layout.block_table[b, pos // layout.page_size].astype(np.int64) * layout.page_size + pos % layout.page_size
    K, KS, V, VS = decoded.tokens(slots)
    stats.add(flip_tolerant(K, KS, k_rot, ("history key", b), max_per_row=1))
    stats.add(flip_tolerant(V, VS, v_rot, ("history value", b), max_per_row=1))
    c.k_codes[:L], c.k_scales[:L] = K, KS
    c.v_codes[:L], c.v_scales[:L] = V, VS
    return c


def block_tolerance(ref):
    """Acceptance bound of a block output: 2e-3 * max|oracle| + 1e-3."""
    return 2e-3 * float(np.max(np.abs(ref))) + 1e-3


class BlockCase:
    """Inputs of one decode-block workload (host, numpy)."""

    def __init__(self, wl: W.Workload, seed=0, layer=0, spare_pages=3, x_scale=1.0):
        """x_scale: a power of two multiplying the block input (keeps its bf16
        values exact), to move the RMS of the rows away from 1."""
        self.wl, self.seed, self.layer = wl, seed, layer
        self.dims = wl.dims
        self.lens = wl.cached_lengths(seed)
        self.layout = W.page_layout(wl, self.lens, extra_tokens=1, seed=seed, spare_pages=spare_pages)
        self.w = W.block_weights(wl, layer, seed)
        self.x = (W.hidden_state(wl, seed) * np.float32(x_scale)).astype(np.float32)
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
        oracle's own quantization is a rounding-boundary case (flip_tolerant,
        at most one flipped code per (token, KV head) row)."""
        d = self.dims
        slots = np.array([self.layout.slot(b, int(L)) for b, L in enumerate(self.lens)], np.int32)
        K, KS, V, VS = self.gpu_decoded.tokens(slots)
        self.kv_flips = FlipStats()

        def hook(b, kc, ks, vc, vs, k_rot, v_rot):
            for got_q, got_s, x in ((K[b], KS[b], k_rot), (V[b], VS[b], v_rot)):
                self.kv_flips.add(flip_tolerant(got_q, got_s, np.asarray(x, np.float64), ("new token", b),
                                                max_frac=1.0, max_per_row=1))
            return K[b].astype(kc.dtype), KS[b].astype(ks.dtype), V[b].astype(vc.dtype), VS[b].astype(vs.dtype)

        return hook

    def run_oracle(self, gpu_codes=True):
        """The oracle block; with gpu_codes (after run_gpu), boundary-case
        codes of the history (oracle_history) and of the new token
        (gpu_kv_hook) follow the GPU's choice."""
        d = self.dims
        t0 = time.time()
        qw = oracle.quantize_block_weights(self.w, d)
        host = getattr(self, "gpu_cache", None) if gpu_codes else None
        self.gpu_decoded = DecodedCache(host, d, self.layout.num_pages) if host is not None else None
        self.hist_flips = FlipStats()
        caches = []
        for b, (k, v) in enumerate(self.hist):
            caches.append(oracle_history(self.gpu_decoded, d, self.layout, b, k, v, int(self.lens[b]) + 1,
                                         self.hist_flips))
            if b % 8 == 7:
                say("oracle history", b + 1, "of", len(self.hist), "sequences")
        diag = {}
        hook = self.gpu_kv_hook() if host is not None else None
        y = oracle.decode_block(self.x, qw, caches, self.lens, d, diag=diag, kv_hook=hook)
        if hook is not None:
            say("boundary decisions taken from the GPU: history", self.hist_flips, "; new token", self.kv_flips)
        self.oracle_caches, self.diag = caches, diag
        say("oracle done in %.1fs" % (time.time() - t0))
        return y
