"""Benchmark of the INT4 decode block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 8b-b1]
                    [--phase all|block|dominant|copy|stages|read|fp8]
                    [--no-sweep] [--no-cpu-baseline]

Workloads: 8b-b<B>, 8b-ragged-b<B>, 70b-b<B>, tiny-b<B> (one block), and
step-b<B> (the full 32-layer step, its own JSON line in ms/step).

One step = one decode block (RMSNorm -> INT4 QKV -> RoPE + Hadamard + INT4
append -> split-sequence attention -> O + residual -> RMSNorm -> INT4
gate/up + SwiGLU -> INT4 down + residual) over one batch of synthetic inputs
already resident in HBM.  Steps cycle through several independent layer
instances (own weights, own KV cache) so that the 256 MB Infinity Cache
cannot hold the weights between steps; the chain is replayed from a HIP
graph and timed with events on the stream it runs on.  Prints one JSON line.

The default run (the 8B block at batch 1, 2048 cached tokens) reports:
  value            us per block;
  block_roofline   the headline fraction: the block's algorithmic bytes
                   (packed INT4 weights + fp16 scales + INT4 KV read and
                   append + fp32 residual in and out) per block time, against
                   8 TB/s and against the measured streaming read;
  roofline         kernel-level evidence for the dominant kernel, the gate/up
                   projection with its SwiGLU epilogue: its algorithmic bytes
                   per average launch time (replayed alone from a graph), and
                   `traffic` from the committed rocprofv3 counter summary while
                   that was taken on the current kernel sources;
  measured_peak_GBps  a plain streaming read of 1 GiB (futx_stream_read);
  sweep            block us, bytes and fractions for the ragged 8B blocks at
                   batch 1/4/8/16/32, the 70B block at batch 1/8/32 and the
                   full 8B step at batch 1/16 (weights and caches drawn on the
                   device from a seeded generator with the workloads'
                   distributions: the timing does not depend on the values);
  cpu_baseline     the fp64 oracle on the host (see cpu_baseline()).

--phase dominant runs only the gate/up stage (counter collection), --phase
copy a plain device copy of known size (counter calibration), --phase read
the streaming read alone, --phase stages every stage of the block alone,
--phase fp8 the 8B projections as INT4 and as FP8 (e4m3) side by side.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "INT4 decode-block µs/step and % of HBM roofline, 8B/70B shapes, batch 1-32"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
DOMINANT = "int4_gemm_kernel, gate/up projection + SwiGLU epilogue"
# sources of the dominant kernel; a counter summary counts only for these exact bytes
KERNEL_SOURCES = ["int4_weight_kv_amd/csrc/gemm.hip", "int4_weight_kv_amd/csrc/gemm.h",
                  "int4_weight_kv_amd/csrc/device.h", "int4_weight_kv_amd/csrc/layout.h"]
COUNTERS_FILE = "profiles/gateup_swiglu_8b_b1_counters.txt"
COPY_BYTES = 512 << 20
READ_BYTES = 1 << 30
READ_POOL = 4 << 30  # the reads cycle over this much memory (beyond the Infinity Cache)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def workload_by_name(name):
    from int4_weight_kv_amd import workload as W

    kind, b = name.rsplit("-b", 1)
    b = int(b)
    if kind == "8b":
        return W.llama8b(b), "Llama-3.1-8B-shape decode block, 2048 cached tokens"
    if kind == "8b-ragged":
        return W.llama8b_ragged(b), "Llama-3.1-8B-shape decode block, ragged 512-4096 cached tokens, outlier keys"
    if kind == "70b":
        return W.llama70b(b), "Llama-3-70B-shape decode block, 4096 cached tokens"
    if kind == "tiny":
        return W.tiny(b), "tiny Llama-style decode block, 128 cached tokens"
    if kind == "step":
        return (W.llama8b_full_step(b), "full 32-layer Llama-3.1-8B-shape decode step (embedding, 32 INT4 blocks, "
                "bf16 LM head vocab 128256 + top-1), 8192 cached tokens, outlier keys")
    raise SystemExit(f"unknown workload {name}")


def weight_bytes(n, k, group):
    """Packed INT4 codes + fp16 group scales of an [n][k] projection."""
    return n * k // 2 + n * (k // group) * 2


def algorithmic_bytes(dims, lens):
    """Bytes the block must move: packed INT4 weights + fp16 group scales,
    the INT4 KV cache read (cached tokens + the new one; codes + fp16 scale
    per token per KV head, keys and values), the KV append, fp32 residual in
    and out."""
    d = dims
    g = d.w_group
    weights = (weight_bytes(d.n_qkv, d.hidden, g) + weight_bytes(d.hidden, d.n_heads * d.head_dim, g) +
               weight_bytes(2 * d.intermediate, d.hidden, g) + weight_bytes(d.hidden, d.intermediate, g))
    per_tok = d.n_kv_heads * 2 * (d.head_dim // 2 + 2)
    kv_read = int(np.sum(np.asarray(lens, np.int64) + 1)) * per_tok
    kv_write = len(lens) * per_tok
    resid = 8 * len(lens) * d.hidden
    return weights + kv_read + kv_write + resid


def gateup_bytes(dims, batch):
    """Algorithmic bytes of one gate/up + SwiGLU launch: weights and scales,
    fp32 input rows (read once), bf16 SwiGLU output rows."""
    d = dims
    return weight_bytes(2 * d.intermediate, d.hidden, d.w_group) + 4 * batch * d.hidden + 2 * batch * d.intermediate


def step_bytes_full(wl, lens):
    """Algorithmic bytes of a full step: every block's bytes, the embedding
    rows read (bf16), the bf16 LM head, the logits written (fp32)."""
    d = wl.dims
    return (wl.n_layers * algorithmic_bytes(d, lens) + 2 * wl.batch * d.hidden +
            2 * wl.vocab * d.hidden + 4 * wl.batch * wl.vocab)


def source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(bytes_per_launch):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary: FETCH_SIZE + WRITE_SIZE (KiB per dispatch), each scaled by the
    ratio of known bytes to what the same counter reads for a plain copy.
    None when there is no summary or it was taken on other kernel sources."""
    path = os.path.join(ROOT, COUNTERS_FILE)
    if not os.path.exists(path):
        return None, "no counter summary"
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_hash():
        return None, "counter summary taken on other kernel sources"
    try:
        fetch = float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_scale"])
        write = float(kv["write_kib_per_dispatch"]) * float(kv["write_scale"])
    except (KeyError, ValueError):
        return None, "counter summary incomplete"
    return int(round((fetch + write) * 1024)), "rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated"


def frac_fields(nbytes, us, measured_gbps):
    gbps = nbytes / (us * 1e-6) / 1e9
    out = {"GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBS, 4)}
    if measured_gbps:
        out["frac_of_measured_read"] = round(gbps / measured_gbps, 4)
    return out


# ------------------------------------------------------------------ CPU baseline


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_block_setup(wl, layer=0):
    import oracle
    from int4_weight_kv_amd import workload as W

    d = wl.dims
    lens = wl.cached_lengths(0)
    t0 = time.time()
    qw = oracle.quantize_block_weights(W.block_weights(wl, layer), d)
    for name in ("qkv", "o", "gate", "up", "down"):
        qw.dense(name)
    prep = time.time() - t0
    caches = []
    for b, L in enumerate(lens):
        k, v = W.history(wl, layer, b, int(L))
        c = oracle.LogicalKVCache.empty(int(L) + 1, d.n_kv_heads, d.head_dim)
        if L:
            oracle.history_fill(c, k, v, np.arange(int(L)), d)
        caches.append(c)
    return qw, caches, lens, W.hidden_state(wl), prep


def _time_oracle_block(wl, setup, budget_s, max_reps=20):
    import oracle

    qw, caches, lens, x, _ = setup
    times = []
    while len(times) < 3 or (sum(times) < budget_s and len(times) < max_reps):
        t = time.time()
        oracle.decode_block(x, qw, caches, lens, wl.dims)
        times.append(time.time() - t)
    return float(np.median(times)), len(times)


def cpu_baseline(wl, budget_s=15.0):
    """The CPU oracle (fp64 numpy, numpy's BLAS) on the host, never tuned:
    one block of the headline workload with every core available to the
    process, the same with one thread, the tiny block, and an estimate of the
    full 32-layer 8B step at 8192 cached tokens (one layer timed, plus the LM
    head on a slice of the vocabulary, scaled)."""
    import oracle
    from int4_weight_kv_amd import workload as W
    from threadpoolctl import threadpool_info, threadpool_limits

    cores = len(os.sched_getaffinity(0))
    out = {"unit": "us/step", "kind": "oracle", "cpu_model": _cpu_model()}
    setup = _oracle_block_setup(wl)
    with threadpool_limits(cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        med, n = _time_oracle_block(wl, setup, budget_s)
    out.update(value=round(med * 1e6, 1), cores=int(used),
               sample=f"{n} block forwards of the same workload (weights pre-dequantized to fp64 in "
                      f"{setup[4]:.1f} s, not timed), median")
    with threadpool_limits(1):
        med1, n1 = _time_oracle_block(wl, setup, budget_s / 3, max_reps=5)
        tiny = W.tiny(1)
        ts = _oracle_block_setup(tiny)
        med0, _ = _time_oracle_block(tiny, ts, 1.0)
    out["one_thread_us"] = round(med1 * 1e6, 1)
    out["tiny_block_one_thread_us"] = round(med0 * 1e6, 1)
    del setup
    # full step estimate: one layer at 8192 cached tokens, the head on 1/8 of the vocabulary
    step = W.llama8b_full_step(1)
    ss = _oracle_block_setup(step)
    with threadpool_limits(cores):
        med_l, _ = _time_oracle_block(step, ss, 3.0, max_reps=3)
        emb, head, gain = W.lm_tables(W.Workload(step.name, step.dims, 1, step.lengths, vocab=16032), 0)
        folded = oracle.fold_head(head, gain)
        x = emb[:1].astype(np.float32)
        t = time.time()
        oracle.lm_head(x, folded, step.dims.rms_eps)
        head_s = (time.time() - t) * step.vocab / 16032
    out["full_step_estimate_ms"] = round((step.n_layers * med_l + head_s) * 1e3, 1)
    out["full_step_sample"] = ("one 8B layer at 8192 cached tokens timed (x 32) plus the fp64 LM head on "
                               "16032 of 128256 rows (scaled)")
    return out


# ------------------------------------------------------------------ device setup


def _device_weights(torch, dims, w_std, seed, outliers):
    """One block's fp32 weights drawn on the device from a seeded generator
    (the workloads' distributions: N(0, w_std) weights, U[0.5, 1.5] gains,
    4 x16 key channels per KV head when `outliers`), returned as host
    arrays for the packer."""
    d = dims
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)

    def normal(*shape):
        return (torch.randn(shape, generator=g, device="cuda") * w_std).cpu().numpy()

    def gain():
        return (torch.rand(d.hidden, generator=g, device="cuda") + 0.5).cpu().numpy()

    w = {"wqkv": normal(d.n_qkv, d.hidden), "wo": normal(d.hidden, d.n_heads * d.head_dim),
         "wgate": normal(d.intermediate, d.hidden), "wup": normal(d.intermediate, d.hidden),
         "wdown": normal(d.hidden, d.intermediate), "gain_attn": gain(), "gain_ffn": gain()}
    if outliers:
        r = np.random.default_rng(seed)
        for h in range(d.n_kv_heads):
            rows = d.n_heads * d.head_dim + h * d.head_dim + np.sort(r.choice(d.head_dim, 4, replace=False))
            w["wqkv"][rows, :] *= np.float32(16.0)
    return w


def _device_cache(torch, DB, dims, layout, lens, seed):
    """A layer's KV cache filled on the device: N(0, 1) keys and values of
    every cached token through futx_kv_append (RoPE + rotation + INT4)."""
    cache = DB.DeviceKVCache(dims, layout.num_pages, zero=False)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    table = torch.from_numpy(layout.block_table).cuda()
    for b, L in enumerate(lens):
        L = int(L)
        if L == 0:
            continue
        k = torch.randn((L, dims.n_kv_heads, dims.head_dim), generator=g, device="cuda")
        v = torch.randn((L, dims.n_kv_heads, dims.head_dim), generator=g, device="cuda")
        pos = torch.arange(L, dtype=torch.int32, device="cuda")
        slots = (table[b, (pos // layout.page_size).long()] * layout.page_size + pos % layout.page_size).int()
        cache.append(k, v, pos, slots)
    return cache


class Timer:
    """Graph capture and event timing on one stream."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.Stream()

    def capture(self, fn, n):
        g = self.torch.cuda.CUDAGraph()
        with self.torch.cuda.graph(g, stream=self.stream):
            for i in range(n):
                fn(i)
        return g

    def run(self, fn, n):
        with self.torch.cuda.stream(self.stream):
            for i in range(n):
                fn(i)
        self.stream.synchronize()

    def timed(self, graphs, reps):
        """Replays `graphs` (list of (graph, count)) `reps` times between two
        events recorded on the stream; returns (ms, count)."""
        torch = self.torch
        for g, _ in graphs:  # one untimed replay
            with torch.cuda.stream(self.stream):
                g.replay()
        self.stream.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        n = 0
        with torch.cuda.stream(self.stream):
            start.record(self.stream)
            for _ in range(reps):
                for g, c in graphs:
                    g.replay()
                    n += c
            stop.record(self.stream)
        stop.synchronize()
        return start.elapsed_time(stop), n


def measure_read(torch, F, timer):
    """GB/s of futx_stream_read over 1 GiB, cycling through 4 GiB so that no
    read hits the Infinity Cache; best of several workgroup counts."""
    pool = torch.empty(READ_POOL, dtype=torch.uint8, device="cuda")
    pool.fill_(1)
    sink = torch.empty(65536, dtype=torch.int32, device="cuda")
    nreg = READ_POOL // READ_BYTES
    best = None
    for wgs in (1024, 2048, 4096):
        fn = lambda i, wgs=wgs: F.futx_stream_read(pool[(i % nreg) * READ_BYTES:], READ_BYTES, sink, wgs,
                                                     timer.stream.cuda_stream)
        g = timer.capture(fn, 2 * nreg)
        ms, n = timer.timed([(g, 2 * nreg)], 3)
        gbps = READ_BYTES * n / (ms * 1e-3) / 1e9
        if best is None or gbps > best[0]:
            best = (gbps, wgs)
    del pool
    torch.cuda.empty_cache()
    return round(best[0], 1), best[1]


def time_blocks(torch, timer, runner, layers, caches, x, reps_blocks):
    """us per block of `runner` cycling the layer instances from a graph."""
    nl = len(layers)
    block = lambda i: runner.decode(layers[i % nl], caches[i % nl], x, timer.stream.cuda_stream)
    timer.run(block, nl)
    g = timer.capture(block, nl)
    reps = max(1, (reps_blocks + nl - 1) // nl)
    ms, n = timer.timed([(g, nl)], reps)
    return ms * 1e3 / n


def sweep(torch, timer, measured, log_every=True):
    """Block times over the metric's batches: the ragged 8B block (batch 1, 4,
    8, 16, 32; 3 layer instances), the 70B block (batch 1, 4, 8, 16, 32; 2
    instances) and the full 8B step (batch 1, 16)."""
    from int4_weight_kv_amd import block as DB
    from int4_weight_kv_amd import workload as W

    out = []
    for name, mk, batches, nl, seed0 in (("8b-ragged", W.llama8b_ragged, (1, 4, 8, 16, 32), 3, 100),
                                         ("70b", W.llama70b, (1, 4, 8, 16, 32), 2, 200)):
        wl0 = mk(1)
        d = wl0.dims
        layers = []
        for li in range(nl):
            layers.append(DB.DeviceLayer(d, _device_weights(torch, d, wl0.w_std, seed0 + li, wl0.outliers)))
        log(f"sweep {name}: {nl} layer instances packed")
        for B in batches:
            wl = mk(B)
            lens = wl.cached_lengths(0)
            layout = W.page_layout(wl, lens, extra_tokens=1, seed=0)
            caches = [_device_cache(torch, DB, d, layout, lens, seed0 + 50 + li) for li in range(nl)]
            runner = DB.DecodeRunner(d, B, lens, layout.block_table)
            x = torch.randn((B, d.hidden), device="cuda")
            us = time_blocks(torch, timer, runner, layers, caches, x, 24)
            nbytes = algorithmic_bytes(d, lens)
            row = {"workload": f"{name}-b{B}", "batch": B, "block_us": round(us, 2), "bytes": int(nbytes)}
            row.update(frac_fields(nbytes, us, measured))
            out.append(row)
            log("sweep", json.dumps(row))
            del caches, runner
            torch.cuda.empty_cache()
        del layers
        torch.cuda.empty_cache()
    out.extend(full_step_sweep(torch, timer, measured))
    return out


def full_step_sweep(torch, timer, measured, batches=(1, 16)):
    """The full 32-layer 8B step (embedding, 32 blocks, final norm + bf16 LM
    head + top-1) at 8192 cached tokens, one graph per batch."""
    from int4_weight_kv_amd import block as DB
    from int4_weight_kv_amd import workload as W

    wl0 = W.llama8b_full_step(1)
    d = wl0.dims
    layers = [DB.DeviceLayer(d, _device_weights(torch, d, wl0.w_std, 300 + li, True)) for li in range(wl0.n_layers)]
    g = torch.Generator(device="cuda")
    g.manual_seed(399)
    tab = lambda: (torch.randn((wl0.vocab, d.hidden), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    emb = tab().float().cpu().numpy()
    head = tab().float().cpu().numpy()
    gain = (torch.rand(d.hidden, generator=g, device="cuda") + 0.5).cpu().numpy()
    log("sweep full step: 32 layers and the LM head ready")
    out = []
    for B in batches:
        wl = W.llama8b_full_step(B)
        lens = wl.cached_lengths(0)
        layout = W.page_layout(wl, lens, extra_tokens=1, seed=0)
        caches = [_device_cache(torch, DB, d, layout, lens, 350 + li) for li in range(wl.n_layers)]
        dh = DB.DecodeHead(d, emb, head, gain, B)
        runner = DB.DecodeRunner(d, B, lens, layout.block_table)
        stepper = DB.DecodeStep(d, layers, caches, dh, runner)
        tok = torch.from_numpy(W.tokens(wl)).cuda()
        x = torch.empty((B, d.hidden), dtype=torch.float32, device="cuda")
        logits = torch.empty((B, wl.vocab), dtype=torch.float32, device="cuda")
        top1 = torch.empty(B, dtype=torch.int32, device="cuda")
        fn = lambda i: stepper.step(tok, x, logits, top1, timer.stream.cuda_stream)
        timer.run(fn, 1)
        gr = timer.capture(fn, 1)
        ms, n = timer.timed([(gr, 1)], 5)
        ms /= n
        nbytes = step_bytes_full(wl, lens)
        row = {"workload": f"step-b{B}", "batch": B, "step_ms": round(ms, 4), "bytes": int(nbytes)}
        row.update(frac_fields(nbytes, ms * 1e3, measured))
        out.append(row)
        log("sweep", json.dumps(row))
        del caches, dh, runner, stepper
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ phases


def fp8_phase(torch, F, timer, batches=(1, 8, 16, 32)):
    """The four 8B projections as INT4 (futx_int4_linear) and as FP8 e4m3
    weights and activations (futx_fp8_linear), us per call, each cycling
    enough weight copies to exceed the Infinity Cache; weights drawn on the
    device (the timing does not depend on the values)."""
    from int4_weight_kv_amd import block as DB
    from int4_weight_kv_amd import workload as W

    d = W.LLAMA8B
    shapes = {"qkv": (d.n_qkv, d.hidden), "o": (d.hidden, d.n_heads * d.head_dim),
              "gateup": (2 * d.intermediate, d.hidden), "down": (d.hidden, d.intermediate)}
    g = torch.Generator(device="cuda")
    g.manual_seed(500)
    res = {"phase": "fp8", "shape": "Llama-3.1-8B projections", "unit": "us", "rows": []}
    for proj, (n, k) in shapes.items():
        w = (torch.randn((n, k), generator=g, device="cuda") * 0.02).cpu().numpy()
        copies = max(3, int(np.ceil(800e6 / (n * k))))
        int4 = [DB.pack_projection(d, proj, w, None) for _ in range(copies)]
        f8 = []
        for _ in range(copies):
            pb, sb = F.futx_fp8_packed_sizes(d, proj)
            p, s_ = DB.device_buffer(pb), DB.device_buffer(sb)
            F.futx_pack_fp8_weights(d, proj, w, None, p, s_)
            f8.append((p, s_))
        for B in batches:
            act = torch.randn((B, k), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
            out = torch.empty((B, n), dtype=torch.float32, device="cuda")
            ws4 = F.futx_decode_workspace_size(d, B, 1)
            ws8 = F.futx_fp8_linear_workspace_size(d, proj, B)
            wsb = DB.device_buffer(max(ws4, ws8))
            st = timer.stream.cuda_stream
            f4 = lambda i: F.futx_int4_linear(d, proj, (int4[i % copies].packed, int4[i % copies].scales), B, act,
                                              out, wsb, ws4, st)
            f8f = lambda i: F.futx_fp8_linear(d, proj, f8[i % copies], B, act, out, wsb, ws8, st)
            row = {"proj": proj, "batch": B, "N": n, "K": k}
            for name, fn, nbytes in (("int4", f4, n * k // 2 + n * (k // 128) * 2),
                                     ("fp8", f8f, n * k + n * (k // 128) * 4)):
                timer.run(fn, copies)
                ms, cnt = timer.timed([(timer.capture(fn, 2 * copies), 2 * copies)], 4)
                us = ms * 1e3 / cnt
                row[name + "_us"] = round(us, 2)
                row[name + "_weight_GBps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
            row["int4_speedup"] = round(row["fp8_us"] / row["int4_us"], 3)
            res["rows"].append(row)
            log("fp8", json.dumps(row))
        del int4, f8
        torch.cuda.empty_cache()
    return res


def full_step_phase(args, wl, desc):
    """Times the full decode step of the workload's own seeded inputs (32
    distinct layers: the weights alone, 3.6 GB, exceed the Infinity Cache)
    replayed from one graph; one JSON line in ms/step."""
    import torch

    from int4_weight_kv_amd import block as DB
    from int4_weight_kv_amd import workload as W

    d = wl.dims
    lens = wl.cached_lengths(0)
    layout = W.page_layout(wl, lens, extra_tokens=1, seed=0)
    layers, caches = [], []
    for li in range(wl.n_layers):
        w = W.block_weights(wl, li)
        layers.append(DB.DeviceLayer(d, w))
        del w
        cache = DB.DeviceKVCache(d, layout.num_pages)
        for b, L in enumerate(lens):
            k, v = W.history(wl, li, b, int(L))
            DB.fill_history(cache, k, v, layout, b)
        caches.append(cache)
        log(f"layer {li} set up")
    emb, head, gain = W.lm_tables(wl)
    dh = DB.DecodeHead(d, emb, head, gain, wl.batch)
    del emb, head
    runner = DB.DecodeRunner(d, wl.batch, lens, layout.block_table)
    step = DB.DecodeStep(d, layers, caches, dh, runner)
    tok = torch.from_numpy(W.tokens(wl)).cuda()
    x = torch.empty((wl.batch, d.hidden), dtype=torch.float32, device="cuda")
    logits = torch.empty((wl.batch, wl.vocab), dtype=torch.float32, device="cuda")
    top1 = torch.empty(wl.batch, dtype=torch.int32, device="cuda")
    timer = Timer(torch)
    fn = lambda i: step.step(tok, x, logits, top1, timer.stream.cuda_stream)
    timer.run(fn, max(1, args.warmup))
    g = timer.capture(fn, 1)
    ms, n = timer.timed([(g, 1)], args.steps)
    ms /= n
    nbytes = step_bytes_full(wl, lens)
    print(json.dumps({
        "metric": "full decode step ms/step (32 INT4 blocks + embedding + bf16 LM head)",
        "value": round(ms, 4), "unit": "ms/step", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": desc, "batch": int(wl.batch), "cached_tokens": int(lens[0]), "graph_replay": True,
                   "step_bytes": int(nbytes), "step_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                   "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }), flush=True)


def copy_phase(torch, reps):
    """A plain device copy of COPY_BYTES, for the counter calibration."""
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"phase": "copy", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES, "reps": reps}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="8b-b1")
    ap.add_argument("--layers", type=int, default=0, help="layer instances cycled (default: enough to exceed MALL)")
    ap.add_argument("--phase", default="all", choices=["all", "block", "dominant", "copy", "stages", "read", "fp8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode path here has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.phase == "copy":
        copy_phase(torch, max(args.steps, 1))
        return

    from int4_weight_kv_amd import block as DB
    from int4_weight_kv_amd import futx as F
    from int4_weight_kv_amd import workload as W

    timer = Timer(torch)
    if args.phase == "read":
        gbps, wgs = measure_read(torch, F, timer)
        print(json.dumps({"phase": "read", "measured_peak_GBps": gbps, "workgroups": wgs, "bytes": READ_BYTES}))
        return

    if args.phase == "fp8":
        print(json.dumps(fp8_phase(torch, F, timer)), flush=True)
        return

    wl, desc = workload_by_name(args.workload)
    if args.workload.startswith("step-"):
        full_step_phase(args, wl, desc)
        return
    measured = None
    if args.phase == "all":
        measured, read_wgs = measure_read(torch, F, timer)
        log(f"streaming read {measured} GB/s")
    d = wl.dims
    lens = wl.cached_lengths(0)
    layout = W.page_layout(wl, lens, extra_tokens=1, seed=0)
    step_bytes = algorithmic_bytes(d, lens)
    # enough independent layers that their weights exceed 2.5x the 256 MB
    # Infinity Cache (6 for the 8B shape, 2 for 70B), at most 8
    nl = args.layers if args.layers > 0 else min(8, max(2, int(np.ceil(640e6 / step_bytes))))
    log(f"{args.workload}: {desc}; {nl} layer instances; setting up")

    layers, caches = [], []
    for li in range(nl):
        w = W.block_weights(wl, li)
        layers.append(DB.DeviceLayer(d, w))
        del w
        cache = DB.DeviceKVCache(d, layout.num_pages)
        for b, L in enumerate(lens):
            k, v = W.history(wl, li, b, int(L))
            DB.fill_history(cache, k, v, layout, b)
        caches.append(cache)
    runner = DB.DecodeRunner(d, wl.batch, lens, layout.block_table)
    x = torch.from_numpy(W.hidden_state(wl)).cuda()
    torch.cuda.synchronize()
    block = lambda i: runner.decode(layers[i % nl], caches[i % nl], x, timer.stream.cuda_stream)
    timer.run(block, max(args.warmup, nl))

    out = {}
    if args.phase in ("all", "block"):
        full, rem = divmod(args.steps, nl)
        ms = 0.0
        if full:
            ms += timer.timed([(timer.capture(block, nl), nl)], full)[0]
        if rem:
            ms += timer.timed([(timer.capture(block, rem), rem)], 1)[0]
        ms_per_step = ms / args.steps
        us = ms_per_step * 1e3
        achieved = step_bytes / (us * 1e-6) / 1e9
        out.update({
            "metric": METRIC,
            "value": round(us, 3),
            "unit": "us/step",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 6),
            "higher_is_better": False,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {
                "workload": desc,
                "batch": int(wl.batch),
                "cached_tokens": [int(v) for v in lens] if len(lens) <= 4 else
                {"min": int(lens.min()), "max": int(lens.max()), "mean": float(lens.mean())},
                "layer_instances_cycled": nl,
                "graph_replay": True,
                "step_bytes": int(step_bytes),
                "step_GBps": round(achieved, 1),
            },
            "block_roofline": {
                "headline": True,
                "bound": "hbm",
                "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "bytes_per_block": int(step_bytes),
                "what": "the whole block: algorithmic bytes per block time",
            },
        })
        if measured:
            out["measured_peak_GBps"] = measured
            out["measured_peak_how"] = (f"futx_stream_read of {READ_BYTES >> 20} MiB cycling over "
                                        f"{READ_POOL >> 30} GiB, {read_wgs} workgroups, graph-replayed")
            out["block_roofline"]["frac_of_measured_read"] = round(achieved / measured, 4)

    if args.phase == "stages":
        # per-stage times (futx_decode_block_stage), each stage replayed alone
        # from a graph over the cycled layers
        names = ["qkv", "attention", "o", "gateup", "down"]
        res = {"phase": "stages", "workload": args.workload, "batch": int(wl.batch), "layers": nl, "unit": "us"}
        ms, n = timer.timed([(timer.capture(block, 4 * nl), 4 * nl)], max(1, args.steps // (4 * nl)))
        res["block"] = round(ms * 1e3 / n, 2)
        for si, nm in enumerate(names):
            fn = lambda i, si=si: runner.stage(layers[i % nl], caches[i % nl], x, si, timer.stream.cuda_stream)
            ms, n = timer.timed([(timer.capture(fn, 4 * nl), 4 * nl)], max(1, args.steps // (4 * nl)))
            res[nm] = round(ms * 1e3 / n, 2)
        res["algorithmic_bytes"] = int(step_bytes)
        res["block_GBps"] = round(step_bytes / (res["block"] * 1e-6) / 1e9, 1)
        print(json.dumps(res), flush=True)
        return

    if args.phase in ("all", "dominant"):
        # the dominant kernel alone: gate/up + SwiGLU stage, cycling layers
        stage = lambda i: runner.stage(layers[i % nl], caches[i % nl], x, F.FUTX_STAGE_GATEUP, timer.stream.cuda_stream)
        per = max(nl, 6 * nl)
        reps = max(1, (args.steps + per - 1) // per)
        ms, n = timer.timed([(timer.capture(stage, per), per)], reps)
        launch_us = ms * 1e3 / n
        nbytes = gateup_bytes(d, wl.batch)
        achieved = nbytes / (launch_us * 1e-6) / 1e9
        traffic, tsrc = read_traffic(nbytes)
        out["roofline"] = {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": DOMINANT,
            "level": "kernel (evidence); the headline fraction is block_roofline",
            "launch_us": round(launch_us, 3),
            "launches_timed": n,
            "bytes_per_launch": int(nbytes),
            "traffic_source": tsrc,
        }
        if measured:
            out["roofline"]["frac_of_measured_read"] = round(achieved / measured, 4)
        if args.phase == "dominant":
            out = {"phase": "dominant", "roofline": out["roofline"]}

    if args.phase == "all":
        del layers, caches, runner
        torch.cuda.empty_cache()
        if not args.no_sweep:
            log("sweep over the metric's batches")
            out["sweep"] = sweep(torch, timer, measured)
        if not args.no_cpu_baseline:
            log("timing the CPU oracle baseline")
            out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
