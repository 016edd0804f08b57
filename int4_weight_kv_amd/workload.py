"""Seeded synthetic inputs for the INT4 decode block.

This module only draws random numbers and lays out inputs; it holds none of
the method's arithmetic (no quantization, rotation, RoPE or attention).  Both
the HIP path and the CPU oracle consume what it returns, so it imports
neither of them.

Every array comes from its own numpy PCG64 stream seeded with
``crc32("futx/<workload>/<layer>/<tensor>")`` plus an optional user seed, so
a tensor is reproducible on its own, in any order.

Shapes (Llama-style blocks):

* tiny:  hidden 256, 4 query / 2 KV heads of 64, SwiGLU 768, weight group 64,
  Hadamard block 32;
* 8B:    hidden 4096, 32 / 8 heads of 128, SwiGLU 14336, group 128, block 64;
* 70B:   hidden 8192, 64 / 8 heads of 128, SwiGLU 28672, group 128, block 64.

Distributions: weights N(0, 0.02) (0.015 for the 70B shape), RMSNorm gains
U[0.5, 1.5] (a unit gain would make gain folding untestable), hidden state
N(0, 1) rounded to bf16, cached pre-RoPE keys and values N(0, 1).  Outlier
workloads scale 4 seeded channels of every KV head by 16, both in the cached
pre-RoPE keys and in the matching W_k rows, so the new token's key carries the
same outliers.  Ragged workloads draw each sequence's cached length
uniformly from [512, 4096]; the pages of all sequences are a seeded
permutation of the pool, so no sequence's pages are contiguous.
"""

import zlib
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

PAGE_SIZE = 64


@dataclass(frozen=True)
class Dims:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    w_group: int
    had_block: int
    page_size: int = PAGE_SIZE
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def n_qkv(self):
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim


TINY = Dims(256, 4, 2, 64, 768, 64, 32)
LLAMA8B = Dims(4096, 32, 8, 128, 14336, 128, 64)
LLAMA70B = Dims(8192, 64, 8, 128, 28672, 128, 64)


@dataclass(frozen=True)
class Workload:
    """One synthetic decode workload (shape, batch and cache lengths)."""

    name: str
    dims: Dims
    batch: int
    lengths: str  # "fixed:<L>" or "uniform:<lo>:<hi>"
    w_std: float = 0.02
    outliers: bool = False
    n_layers: int = 1
    vocab: int = 0  # > 0 for a full step with embedding and LM head

    def cached_lengths(self, seed: int = 0):
        kind, *args = self.lengths.split(":")
        if kind == "fixed":
            return np.full(self.batch, int(args[0]), dtype=np.int32)
        lo, hi = int(args[0]), int(args[1])
        r = rng(self.name, "lengths", "L", seed=seed)
        return r.integers(lo, hi + 1, size=self.batch, dtype=np.int64).astype(np.int32)


def tiny(batch=1, length=128):
    return Workload(f"tiny-b{batch}-L{length}", TINY, batch, f"fixed:{length}")


def llama8b(batch=1, length=2048):
    return Workload(f"8b-b{batch}-L{length}", LLAMA8B, batch, f"fixed:{length}")


def llama8b_ragged(batch):
    return Workload(f"8b-ragged-b{batch}", LLAMA8B, batch, "uniform:512:4096", outliers=True)


def llama70b(batch=1, length=4096):
    return Workload(f"70b-b{batch}-L{length}", LLAMA70B, batch, f"fixed:{length}", w_std=0.015)


def llama8b_full_step(batch=1, length=8192):
    return Workload(f"8b-step-b{batch}-L{length}", LLAMA8B, batch, f"fixed:{length}",
                    outliers=True, n_layers=32, vocab=128256)


def rng(workload: str, layer, tensor: str, seed: int = 0) -> np.random.Generator:
    key = f"futx/{workload}/{layer}/{tensor}"
    return np.random.Generator(np.random.PCG64([zlib.crc32(key.encode()), seed]))


def _normal(r, shape, std):
    out = r.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def to_bf16_values(x32):
    """Round fp32 values to bf16 (torch's cast) and return them as fp32."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def outlier_channels(wl: Workload, layer, seed=0):
    """[n_kv_heads][4] channel indices that carry x16 outliers (or None)."""
    if not wl.outliers:
        return None
    d = wl.dims
    r = rng(wl.name, layer, "outlier_channels", seed)
    return np.stack([np.sort(r.choice(d.head_dim, 4, replace=False)) for _ in range(d.n_kv_heads)])


def block_weights(wl: Workload, layer=0, seed=0):
    """fp32 weights of one block: wqkv, wo, wgate, wup, wdown, gain_attn, gain_ffn."""
    d = wl.dims
    nq_d, nkv_d = d.n_heads * d.head_dim, d.n_kv_heads * d.head_dim
    w = {
        "wqkv": _normal(rng(wl.name, layer, "wqkv", seed), (d.n_qkv, d.hidden), wl.w_std),
        "wo": _normal(rng(wl.name, layer, "wo", seed), (d.hidden, nq_d), wl.w_std),
        "wgate": _normal(rng(wl.name, layer, "wgate", seed), (d.intermediate, d.hidden), wl.w_std),
        "wup": _normal(rng(wl.name, layer, "wup", seed), (d.intermediate, d.hidden), wl.w_std),
        "wdown": _normal(rng(wl.name, layer, "wdown", seed), (d.hidden, d.intermediate), wl.w_std),
        "gain_attn": rng(wl.name, layer, "gain_attn", seed).uniform(0.5, 1.5, d.hidden).astype(np.float32),
        "gain_ffn": rng(wl.name, layer, "gain_ffn", seed).uniform(0.5, 1.5, d.hidden).astype(np.float32),
    }
    oc = outlier_channels(wl, layer, seed)
    if oc is not None:
        for h in range(d.n_kv_heads):
            rows = nq_d + h * d.head_dim + oc[h]
            w["wqkv"][rows, :] *= np.float32(16.0)
    return w


def hidden_state(wl: Workload, seed=0, tag="x"):
    """Block input [B][hidden]: N(0, 1) rounded to bf16, stored as fp32."""
    x = _normal(rng(wl.name, "in", tag, seed), (wl.batch, wl.dims.hidden), 1.0)
    return to_bf16_values(x)


def history(wl: Workload, layer, b, length, seed=0):
    """Pre-RoPE keys and values of the cached tokens of sequence b: fp32 [L][nkv][d]."""
    d = wl.dims
    k = _normal(rng(wl.name, layer, f"k_hist{b}", seed), (length, d.n_kv_heads, d.head_dim), 1.0)
    v = _normal(rng(wl.name, layer, f"v_hist{b}", seed), (length, d.n_kv_heads, d.head_dim), 1.0)
    oc = outlier_channels(wl, layer, seed)
    if oc is not None:
        for h in range(d.n_kv_heads):
            k[:, h, oc[h]] *= np.float32(16.0)
    return k, v


@dataclass
class PageLayout:
    """Block table of a batch: physical page of logical page j of sequence b."""

    block_table: np.ndarray  # int32 [B][max_pages_per_seq], unused entries -1
    num_pages: int
    page_size: int = PAGE_SIZE

    def slot(self, b, t):
        return int(self.block_table[b, t // self.page_size]) * self.page_size + t % self.page_size


def page_layout(wl: Workload, lengths: Sequence[int], extra_tokens=1, seed=0, spare_pages=0):
    """Pages for lengths[b] + extra_tokens tokens per sequence, drawn from a
    seeded permutation of a pool with ``spare_pages`` unused pages."""
    ps = wl.dims.page_size
    need = [(int(L) + extra_tokens + ps - 1) // ps for L in lengths]
    total = sum(need) + spare_pages
    perm = rng(wl.name, "pages", "perm", seed).permutation(total).astype(np.int32)
    mpps = max(need) if need else 1
    table = np.full((len(lengths), mpps), -1, dtype=np.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[at:at + n]
        at += n
    return PageLayout(table, total, ps)


def tokens(wl: Workload, seed=0):
    return rng(wl.name, "in", "tokens", seed).integers(0, wl.vocab, size=wl.batch).astype(np.int32)


def lm_tables(wl: Workload, seed=0):
    """Embedding and LM head: bf16 values (stored as fp32) [vocab][hidden], and the final gain."""
    d = wl.dims
    emb = to_bf16_values(_normal(rng(wl.name, "emb", "table", seed), (wl.vocab, d.hidden), 0.02))
    head = to_bf16_values(_normal(rng(wl.name, "head", "table", seed), (wl.vocab, d.hidden), 0.02))
    gain = rng(wl.name, "head", "gain", seed).uniform(0.5, 1.5, d.hidden).astype(np.float32)
    return emb, head, gain
