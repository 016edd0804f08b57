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
    def run_oracle(self):
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
        y = oracle.decode_block(self.x, qw, caches, self.lens, d, diag=diag)
        self.oracle_caches, self.diag = caches, diag
        say("oracle done in %.1fs" % (time.time() - t0))
        return y
