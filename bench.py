"""Benchmark of the INT4 decode block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 8b-b1]
                    [--phase all|block|dominant|copy]

Workloads: 8b-b<B>, 8b-ragged-b<B>, 70b-b<B>, tiny-b<B> (one block), and
step-b<B> (the full 32-layer step, its own JSON line in ms/step).

One step = one decode block (RMSNorm -> INT4 QKV -> RoPE + Hadamard + INT4
append -> split-sequence attention -> O + residual -> RMSNorm -> INT4
gate/up + SwiGLU -> INT4 down + residual) over one batch of synthetic inputs
already resident in HBM.  Steps cycle through several independent layer
instances (own weights, own KV cache) so that the 256 MB Infinity Cache
cannot hold the weights between steps; the chain is replayed from a HIP
graph.  Prints one JSON line.

The roofline object is for the dominant kernel, the gate/up projection with
its SwiGLU epilogue (about half of the bytes of a step): its stage is
replayed alone from a graph, timed with HIP events on the stream it is
launched on, and its algorithmic bytes per launch (packed weights, fp16
scales, the fp32 input rows and the bf16 output rows) are divided by the
average launch time.  `traffic` comes from the committed rocprofv3 counter
summary of that kernel when it was taken on the current kernel sources.

--phase dominant runs only that stage (for counter collection), --phase copy
a plain device copy of known size (the counter calibration).
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


def cpu_baseline(wl, lens, budget_s=15.0):
    """Times the CPU oracle (fp64 numpy) on one block of the same workload."""
    import oracle
    from int4_weight_kv_amd import workload as W

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    d = wl.dims
    w = W.block_weights(wl, 0)
    x = W.hidden_state(wl)
    t0 = time.time()
    qw = oracle.quantize_block_weights(w, d)
    for name in ("qkv", "o", "gate", "up", "down"):
        qw.dense(name)
    prep_s = time.time() - t0
    caches = []
    for b, L in enumerate(lens):
        k, v = W.history(wl, 0, b, int(L))
        c = oracle.LogicalKVCache.empty(int(L) + 1, d.n_kv_heads, d.head_dim)
        if L:
            oracle.history_fill(c, k, v, np.arange(int(L)), d)
        caches.append(c)
    times = []
    while len(times) < 3 or (sum(times) < budget_s and len(times) < 20):
        t = time.time()
        oracle.decode_block(x, qw, caches, lens, d)
        times.append(time.time() - t)
    med = float(np.median(times))
    return {
        "value": round(med * 1e6, 1),
        "unit": "us/step",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(times)} block forwards of the same workload on the host (fp64 numpy, weights "
                  f"pre-dequantized to fp64 in {prep_s:.1f} s, not timed), median",
    }


def step_bytes_full(wl, lens):
    """Algorithmic bytes of a full step: every block's bytes, the embedding
    rows read (bf16), the bf16 LM head, the logits written (fp32)."""
    d = wl.dims
    return (wl.n_layers * algorithmic_bytes(d, lens) + 2 * wl.batch * d.hidden +
            2 * wl.vocab * d.hidden + 4 * wl.batch * wl.vocab)


def full_step_phase(args, wl, desc):
    """Times the full decode step (32 distinct layers: the weights alone,
    3.6 GB, exceed the Infinity Cache) replayed from one graph."""
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
        print(f"[bench] layer {li} set up", file=sys.stderr, flush=True)
    emb, head, gain = W.lm_tables(wl)
    dh = DB.DecodeHead(d, emb, head, gain, wl.batch)
    del emb, head
    runner = DB.DecodeRunner(d, wl.batch, lens, layout.block_table)
    step = DB.DecodeStep(d, layers, caches, dh, runner)
    tok = torch.from_numpy(W.tokens(wl)).cuda()
    x = torch.empty((wl.batch, d.hidden), dtype=torch.float32, device="cuda")
    logits = torch.empty((wl.batch, wl.vocab), dtype=torch.float32, device="cuda")
    top1 = torch.empty(wl.batch, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup)):
            step.step(tok, x, logits, top1)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step.step(tok, x, logits, top1)
    with torch.cuda.stream(stream):
        g.replay()
    stream.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(args.steps):
            g.replay()
        stop.record(stream)
    stop.synchronize()
    ms = start.elapsed_time(stop) / args.steps
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
    ap.add_argument("--phase", default="all", choices=["all", "block", "dominant", "copy", "stages"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    wl, desc = workload_by_name(args.workload)
    if args.workload.startswith("step-"):
        full_step_phase(args, wl, desc)
        return
    d = wl.dims
    lens = wl.cached_lengths(0)
    layout = W.page_layout(wl, lens, extra_tokens=1, seed=0)
    step_bytes = algorithmic_bytes(d, lens)
    # enough independent layers that their weights exceed 2.5x the 256 MB
    # Infinity Cache (6 for the 8B shape, 2 for 70B), at most 8
    nl = args.layers if args.layers > 0 else min(8, max(2, int(np.ceil(640e6 / step_bytes))))
    print(f"[bench] {args.workload}: {desc}; {nl} layer instances; setting up", file=sys.stderr, flush=True)

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
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i)
        return g

    def timed(graphs, reps):
        """Replays `graphs` (list of (graph, count)) `reps` times between two
        events recorded on `stream`; returns (ms, launches)."""
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        n = 0
        with torch.cuda.stream(stream):
            start.record(stream)
            for _ in range(reps):
                for g, c in graphs:
                    g.replay()
                    n += c
            stop.record(stream)
        stop.synchronize()
        torch.cuda.synchronize()
        return start.elapsed_time(stop), n

    block = lambda i: runner.decode(layers[i % nl], caches[i % nl], x)
    with torch.cuda.stream(stream):
        for i in range(max(args.warmup, nl)):
            block(i)
    stream.synchronize()

    out = {}
    if args.phase in ("all", "block"):
        full, rem = divmod(args.steps, nl)
        gl = []
        if full:
            gl.append((capture(block, nl), nl))
        g_full = gl[0][0] if gl else None
        with torch.cuda.stream(stream):
            for _ in range(2):
                if g_full:
                    g_full.replay()
        stream.synchronize()
        ms_full, n_full = timed(gl, full) if full else (0.0, 0)
        ms_rem = 0.0
        if rem:
            g_rem = capture(block, rem)
            ms_rem, _ = timed([(g_rem, rem)], 1)
        ms = ms_full + ms_rem
        ms_per_step = ms / args.steps
        us = ms_per_step * 1e3
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
                "step_GBps": round(step_bytes / (us * 1e-6) / 1e9, 1),
            },
        })

    if args.phase == "stages":
        # per-stage times (futx_decode_block_stage), each stage replayed alone
        # from a graph over the cycled layers
        names = ["qkv", "attention", "o", "gateup", "down"]
        res = {"phase": "stages", "workload": args.workload, "batch": int(wl.batch), "layers": nl, "unit": "us"}
        g_blk = capture(block, 4 * nl)
        ms, n = timed([(g_blk, 4 * nl)], max(1, args.steps // (4 * nl)))
        res["block"] = round(ms * 1e3 / n, 2)
        for si, nm in enumerate(names):
            fn = lambda i, si=si: runner.stage(layers[i % nl], caches[i % nl], x, si)
            g = capture(fn, 4 * nl)
            with torch.cuda.stream(stream):
                g.replay()
            stream.synchronize()
            ms, n = timed([(g, 4 * nl)], max(1, args.steps // (4 * nl)))
            res[nm] = round(ms * 1e3 / n, 2)
        res["algorithmic_bytes"] = int(step_bytes)
        res["block_GBps"] = round(step_bytes / (res["block"] * 1e-6) / 1e9, 1)
        print(json.dumps(res), flush=True)
        return

    if args.phase in ("all", "dominant"):
        # the dominant kernel alone: gate/up + SwiGLU stage, cycling layers
        stage = lambda i: runner.stage(layers[i % nl], caches[i % nl], x, F.FUTX_STAGE_GATEUP)
        per = max(nl, 6 * nl)
        g_dom = capture(stage, per)
        with torch.cuda.stream(stream):
            g_dom.replay()
        stream.synchronize()
        reps = max(1, (args.steps + per - 1) // per)
        ms, n = timed([(g_dom, per)], reps)
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
            "launch_us": round(launch_us, 3),
            "launches_timed": n,
            "bytes_per_launch": int(nbytes),
            "traffic_source": tsrc,
        }
        if args.phase == "dominant":
            out = {"phase": "dominant", "roofline": out["roofline"]}

    if args.phase == "all" and not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, lens, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
