"""Device-side setup around the C ABI: packed weights, a paged INT4 KV cache
and a workspace in torch-allocated device memory, and a thin `decode` call.

Everything computational goes through libfutx.so (futx.py); torch only
allocates memory and provides the stream.
"""

from dataclasses import dataclass

import numpy as np

from . import futx as F


def _torch():
    import torch

    return torch


def device_buffer(nbytes, device="cuda"):
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


@dataclass
class PackedProj:
    packed: object  # torch uint8 device tensor
    scales: object


def pack_projection(dims, proj, w, gain=None, device="cuda", stream=None):
    pb, sb = F.futx_packed_sizes(dims, proj)
    p = device_buffer(pb, device)
    s = device_buffer(sb, device)
    F.futx_pack_weights(dims, proj, w, gain, p, s, stream)
    return PackedProj(p, s)


class DeviceLayer:
    """One block's packed weights (device)."""

    def __init__(self, dims, w, device="cuda", stream=None):
        self.dims = dims
        self.qkv = pack_projection(dims, "qkv", w["wqkv"], w["gain_attn"], device, stream)
        self.o = pack_projection(dims, "o", w["wo"], None, device, stream)
        self.gateup = pack_projection(dims, "gateup", np.concatenate([w["wgate"], w["wup"]]), w["gain_ffn"], device,
                                      stream)
        self.down = pack_projection(dims, "down", w["wdown"], None, device, stream)
        self.c_weights = F.make_block_weights(*((p.packed, p.scales) for p in (self.qkv, self.o, self.gateup,
                                                                              self.down)))

    @property
    def weight_bytes(self):
        return sum(p.packed.numel() + p.scales.numel() for p in (self.qkv, self.o, self.gateup, self.down))


class DeviceKVCache:
    """A paged INT4 KV cache of one layer (device)."""

    def __init__(self, dims, num_pages, device="cuda", zero=True):
        self.dims = dims
        self.num_pages = int(num_pages)
        cb, sb = F.futx_kv_cache_sizes(dims, num_pages)
        self.k_codes = device_buffer(cb, device)
        self.v_codes = device_buffer(cb, device)
        self.k_scales = device_buffer(sb, device)
        self.v_scales = device_buffer(sb, device)
        if zero:
            for t in (self.k_codes, self.v_codes, self.k_scales, self.v_scales):
                t.zero_()
        self.c_cache = F.make_cache(self.k_codes, self.v_codes, self.k_scales, self.v_scales, num_pages)

    def append(self, k, v, positions, slots, flags=F.FUTX_KV_ROPE | F.FUTX_KV_HADAMARD, stream=None):
        """k, v: device fp32 [n][nkv][d]; positions, slots: device int32 [n]."""
        F.futx_kv_append(self.dims, k.shape[0], k, v, positions, slots, flags, self.c_cache, stream)

    def host_copy(self):
        return tuple(t.cpu().numpy() for t in (self.k_codes, self.v_codes, self.k_scales, self.v_scales))


def fill_history(cache, k_hist, v_hist, layout, b, device="cuda", stream=None, chunk=1 << 16):
    """Writes the first len(k_hist) tokens of sequence b (positions 0..L-1)."""
    torch = _torch()
    L = k_hist.shape[0]
    if L == 0:
        return
    for t0 in range(0, L, chunk):
        t1 = min(L, t0 + chunk)
        pos = np.arange(t0, t1, dtype=np.int32)
        slots = (layout.block_table[b, pos // layout.page_size] * layout.page_size
                 + pos % layout.page_size).astype(np.int32)
        kd = torch.from_numpy(np.ascontiguousarray(k_hist[t0:t1])).to(device)
        vd = torch.from_numpy(np.ascontiguousarray(v_hist[t0:t1])).to(device)
        cache.append(kd, vd, torch.from_numpy(pos).to(device), torch.from_numpy(slots).to(device), stream=stream)


class DecodeRunner:
    """Workspace and metadata for futx_decode_block on one batch."""

    def __init__(self, dims, batch, cached_lens, block_table, device="cuda"):
        torch = _torch()
        self.dims = dims
        self.batch = int(batch)
        self.max_context = int(np.max(cached_lens)) + 1
        self.block_table = torch.from_numpy(np.ascontiguousarray(block_table, np.int32)).to(device)
        self.mpps = int(block_table.shape[1])
        self.cached_lens = torch.from_numpy(np.ascontiguousarray(cached_lens, np.int32)).to(device)
        self.ws_bytes = F.futx_decode_workspace_size(dims, self.batch, self.max_context)
        self.workspace = device_buffer(self.ws_bytes, device)

    def decode(self, layer, cache, x, stream=None):
        """x: device fp32 [B][hidden], updated in place."""
        F.futx_decode_block(self.dims, layer.c_weights, self.batch, x, self.cached_lens, self.block_table,
                            self.mpps, self.max_context, cache.c_cache, self.workspace, self.ws_bytes, stream)

    def stage(self, layer, cache, x, stage, stream=None):
        """One stage of the block (futx_decode_block_stage), for timing."""
        F.futx_decode_block_stage(self.dims, layer.c_weights, self.batch, x, self.cached_lens, self.block_table,
                                  self.mpps, self.max_context, cache.c_cache, self.workspace, self.ws_bytes, stage,
                                  stream)


def bf16_bits(values):
    """bf16 bit patterns of fp32 values, rounded to nearest even (values that
    are already bf16 keep their bits; NaN stays NaN)."""
    u = np.ascontiguousarray(values, np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + (0x7FFF + ((u >> 16) & 1))) >> 16).astype(np.uint16)
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)


class DecodeHead:
    """Embedding table and LM head (final norm gain folded in, bf16) on the device."""

    def __init__(self, dims, emb_values, head_values, final_gain, max_batch, device="cuda"):
        torch = _torch()
        self.dims = dims
        self.vocab, hidden = emb_values.shape
        emb_bits = bf16_bits(emb_values)
        head_bits = bf16_bits(head_values)
        folded = np.empty_like(head_bits)
        F.futx_fold_head(self.vocab, hidden, head_bits, final_gain, folded)
        self.emb = torch.from_numpy(emb_bits.view(np.int16)).to(device)
        self.head = torch.from_numpy(folded.view(np.int16)).to(device)
        self.ws_bytes = F.futx_lm_head_workspace_size(dims, self.vocab, max_batch)
        self.workspace = device_buffer(self.ws_bytes, device)

    def embed(self, tokens, x, stream=None):
        F.futx_embed(self.dims.hidden, self.vocab, self.emb, tokens, tokens.shape[0], x, stream)

    def lm_head(self, x, logits, top1, stream=None):
        F.futx_lm_head(self.dims, self.vocab, self.head, x.shape[0], x, logits, top1, self.workspace,
                       self.ws_bytes, stream)


class DecodeStep:
    """A full decode step: embedding, the blocks in order, final norm + LM head."""

    def __init__(self, dims, layers, caches, head: DecodeHead, runner: DecodeRunner):
        self.dims, self.layers, self.caches, self.head, self.runner = dims, layers, caches, head, runner

    def step(self, tokens, x, logits, top1, stream=None, progress=None):
        """tokens: device int32 [B]; x: device fp32 [B][hidden] scratch; logits fp32 [B][vocab]; top1 int32 [B]."""
        self.head.embed(tokens, x, stream)
        for i, (layer, cache) in enumerate(zip(self.layers, self.caches)):
            self.runner.decode(layer, cache, x, stream)
            if progress is not None:
                progress(i)
        self.head.lm_head(x, logits, top1, stream)


class PagedTable:
    """Host bookkeeping of a paged KV cache shared by the layers of a model:
    a free list of physical pages, the block table [batch][max_pages_per_seq]
    (-1 = no page) and the tokens cached per sequence.  A sequence takes a
    page from the free list when it first needs a position on it, so prompts
    of any length sit unpadded and decode steps grow the table one page at a
    time; release() returns a sequence's pages."""

    def __init__(self, num_pages, batch, max_pages_per_seq, page_size=64, seed=None):
        order = np.arange(num_pages, dtype=np.int32)
        if seed is not None:
            order = np.random.default_rng(seed).permutation(num_pages).astype(np.int32)
        self.free = list(order[::-1])  # taken from the end: the first page taken is order[0]
        self.page_size = page_size
        self.table = np.full((batch, max_pages_per_seq), -1, np.int32)
        self.lens = np.zeros(batch, np.int32)
        self.dirty = True

    def ensure(self, b, n_tokens):
        """Pages for positions 0..n_tokens-1 of sequence b."""
        need = (int(n_tokens) + self.page_size - 1) // self.page_size
        if need > self.table.shape[1]:
            raise RuntimeError(f"sequence {b}: {n_tokens} tokens exceed the block table")
        for j in range(need):
            if self.table[b, j] < 0:
                if not self.free:
                    raise RuntimeError("KV cache out of pages")
                self.table[b, j] = self.free.pop()
                self.dirty = True

    def slots(self, b, positions):
        positions = np.asarray(positions, np.int64)
        return (self.table[b, positions // self.page_size].astype(np.int64) * self.page_size
                + positions % self.page_size).astype(np.int32)

    def release(self, b):
        for j in range(self.table.shape[1]):
            if self.table[b, j] >= 0:
                self.free.append(self.table[b, j])
                self.table[b, j] = -1
        self.lens[b] = 0
        self.dirty = True


class DecodeSession:
    """Token-by-token generation for a batch of sequences: unpadded prompts
    placed in the paged INT4 caches of every layer (futx_kv_append: RoPE,
    rotation, INT4 at their own positions), then decode steps that take cache
    pages as sequences cross page boundaries, run the embedding, every block
    and the LM head through the C ABI, and feed the top-1 token of each
    sequence back as its next input without leaving the device."""

    def __init__(self, dims, layers, head, batch, num_pages, max_context, page_seed=None, device="cuda"):
        torch = _torch()
        self.dims, self.layers, self.head, self.batch = dims, layers, head, int(batch)
        self.max_context = int(max_context)
        mpps = (self.max_context + dims.page_size - 1) // dims.page_size
        self.paged = PagedTable(num_pages, batch, mpps, dims.page_size, page_seed)
        self.caches = [DeviceKVCache(dims, num_pages, device) for _ in layers]
        self.table_d = torch.empty((batch, mpps), dtype=torch.int32, device=device)
        self.lens_d = torch.empty(batch, dtype=torch.int32, device=device)
        self.ws_bytes = F.futx_decode_workspace_size(dims, batch, self.max_context)
        self.workspace = device_buffer(self.ws_bytes, device)
        self.x = torch.empty((batch, dims.hidden), dtype=torch.float32, device=device)
        self.logits = torch.empty((batch, head.vocab), dtype=torch.float32, device=device)
        self.top1 = torch.empty(batch, dtype=torch.int32, device=device)
        self.device = device

    def _sync_metadata(self):
        torch = _torch()
        if self.paged.dirty:
            self.table_d.copy_(torch.from_numpy(self.paged.table))
            self.paged.dirty = False
        self.lens_d.copy_(torch.from_numpy(self.paged.lens))

    def place_prompt(self, b, k_layers, v_layers):
        """Prompt of sequence b: pre-RoPE keys and values [L][nkv][d] (fp32,
        host) of every layer, written at positions 0..L-1."""
        torch = _torch()
        L = int(k_layers[0].shape[0])
        if L + 1 > self.max_context:
            raise ValueError("prompt longer than the session's context")
        self.paged.ensure(b, L)
        self.paged.lens[b] = L
        if L == 0:
            return
        pos = np.arange(L, dtype=np.int32)
        pos_d = torch.from_numpy(pos).to(self.device)
        slots_d = torch.from_numpy(self.paged.slots(b, pos)).to(self.device)
        for cache, k, v in zip(self.caches, k_layers, v_layers):
            cache.append(torch.from_numpy(np.ascontiguousarray(k, np.float32)).to(self.device),
                         torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(self.device), pos_d, slots_d)

    def step(self, tokens, progress=None):
        """One decode step for every sequence: tokens int32 [batch] (device).
        Returns the top-1 tokens (device, the next step's input); the logits
        stay in self.logits.  progress(i, x) runs after block i."""
        for b in range(self.batch):
            self.paged.ensure(b, int(self.paged.lens[b]) + 1)
        if int(self.paged.lens.max()) + 1 > self.max_context:
            raise RuntimeError("a sequence outgrew the session's context")
        self._sync_metadata()
        d = self.dims
        self.head.embed(tokens, self.x)
        mpps = self.paged.table.shape[1]
        for i, (layer, cache) in enumerate(zip(self.layers, self.caches)):
            F.futx_decode_block(d, layer.c_weights, self.batch, self.x, self.lens_d, self.table_d, mpps,
                                self.max_context, cache.c_cache, self.workspace, self.ws_bytes)
            if progress is not None:
                progress(i, self.x)
        self.head.lm_head(self.x, self.logits, self.top1)
        self.paged.lens += 1
        return self.top1
