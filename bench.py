"""Benchmark of the INT4 decode block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 8b-b1]

One step = one decode block (RMSNorm -> INT4 QKV -> RoPE + Hadamard + INT4
append -> split-sequence attention -> O + residual -> RMSNorm -> INT4
gate/up + SwiGLU -> INT4 down + residual) over one batch of synthetic
inputs already resident in HBM.  Steps cycle through several independent
layer instances (own weights, own KV cache) so that the 256 MB Infinity
Cache cannot hold the weights between steps; the whole chain is replayed
from a HIP graph.  Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "INT4 decode-block µs/step and % of HBM roofline, 8B/70B shapes, batch 1-32"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


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
    raise SystemExit(f"unknown workload {name}")


def algorithmic_bytes(dims, lens):
    """Bytes the block must move: packed INT4 weights + fp16 group scales,
    the INT4 KV cache read (cached tokens + the new one; codes + fp16 scale
    per token per KV head, keys and values), the KV append, fp32 residual in
    and out."""
    d = dims
    w_elems = (d.n_qkv * d.hidden + d.hidden * d.n_heads * d.head_dim + 2 * d.intermediate * d.hidden
               + d.hidden * d.intermediate)
    weights = w_elems // 2 + (w_elems // d.w_group) * 2
    per_tok = d.n_kv_heads * 2 * (d.head_dim // 2 + 2)
    kv_read = int(np.sum(np.asarray(lens, np.int64) + 1)) * per_tok
    kv_write = len(lens) * per_tok
    resid = 8 * len(lens) * d.hidden
    return weights + kv_read + kv_write + resid


def cpu_baseline(wl, lens, layout_unused, budget_s=15.0):
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="8b-b1")
    ap.add_argument("--layers", type=int, default=0, help="layer instances cycled (default: enough to exceed MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from int4_weight_kv_amd import block as DB
    from int4_weight_kv_amd import workload as W

    wl, desc = workload_by_name(args.workload)
    d = wl.dims
    lens = wl.cached_lengths(0)
    layout = W.page_layout(wl, lens, extra_tokens=1, seed=0)
    w_bytes_layer = algorithmic_bytes(d, lens)
    # enough independent layers that their weights exceed 2.5x the 256 MB
    # Infinity Cache (6 for the 8B shape, 2 for 70B), at most 8
    nl = args.layers if args.layers > 0 else min(8, max(2, int(np.ceil(640e6 / w_bytes_layer))))
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
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            runner.decode(layers[i % nl], caches[i % nl], x)
    stream.synchronize()

    # graphs: one with nl blocks, one with the remainder
    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                runner.decode(layers[i % nl], caches[i % nl], x)
        return g

    full, rem = divmod(args.steps, nl)
    g_full = capture(nl) if full else None
    g_rem = capture(rem) if rem else None
    with torch.cuda.stream(stream):
        for _ in range(2):
            if g_full:
                g_full.replay()
    stream.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(full):
            g_full.replay()
        if g_rem:
            g_rem.replay()
        stop.record(stream)
    stop.synchronize()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop)
    ms_per_step = ms / args.steps
    us = ms_per_step * 1e3
    achieved = w_bytes_layer / (us * 1e-6) / 1e9

    out = {
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
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "decode block (all kernels of one step)",
            "bytes_per_step": int(w_bytes_layer),
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, lens, layout, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
