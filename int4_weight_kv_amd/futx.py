"""ctypes binding of libfutx.so: the C ABI of include/futx.h, one Python
function per entry point with the same name.

Only argument marshalling lives here: torch tensors (device memory, created
by the caller) and numpy arrays (host memory) are turned into pointers, and
a non-zero status becomes a FutxError.  Every step of the decode block runs
in the HIP kernels of the library.  Importing this module fails loudly if the
library has not been built (there is no fallback).
"""

import ctypes
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfutx.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m int4_weight_kv_amd._build` "
                      "(or __graft_entry__.build()); there is no CPU fallback")
_lib = ctypes.CDLL(_LIB_PATH)

FUTX_OK = 0
FUTX_E_ARG = -1
FUTX_E_UNSUPPORTED = -2
FUTX_E_WORKSPACE = -3
FUTX_E_RANGE = -4
FUTX_E_HIP = -5

FUTX_PROJ_QKV, FUTX_PROJ_O, FUTX_PROJ_GATEUP, FUTX_PROJ_DOWN = 0, 1, 2, 3
PROJ_BY_NAME = {"qkv": 0, "o": 1, "gateup": 2, "down": 3}

# stages of futx_decode_block (futx_decode_block_stage)
(FUTX_STAGE_QKV, FUTX_STAGE_ATTENTION, FUTX_STAGE_O, FUTX_STAGE_GATEUP, FUTX_STAGE_DOWN) = range(5)
FUTX_STAGE_COUNT = 5

FUTX_KV_ROPE = 1
FUTX_KV_HADAMARD = 2

LIBRARY_PATH = _LIB_PATH


class futx_dims(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("w_group", ctypes.c_int32),
        ("had_block", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("rope_theta", ctypes.c_float),
    ]


class futx_qweight(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class futx_block_weights(ctypes.Structure):
    _fields_ = [("qkv", futx_qweight), ("o", futx_qweight), ("gateup", futx_qweight), ("down", futx_qweight)]


class futx_kv_cache(ctypes.Structure):
    _fields_ = [
        ("k_codes", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
    ]


class FutxError(RuntimeError):
    def __init__(self, name, status, message):
        super().__init__(f"{name} failed with status {status}: {message}")
        self.status = status


_P = ctypes.c_void_p
_SZ = ctypes.POINTER(ctypes.c_size_t)
_D = ctypes.POINTER(futx_dims)
_I32 = ctypes.c_int32

_SIGS = {
    "futx_last_error": (ctypes.c_char_p, []),
    "futx_packed_sizes": (_I32, [_D, _I32, _SZ, _SZ]),
    "futx_pack_weights": (_I32, [_D, _I32, _P, _P, _P, _P, _P]),
    "futx_pack_weights_host": (_I32, [_D, _I32, _P, _P, _P, _P]),
    "futx_pack_codes": (_I32, [_D, _I32, _P, _P, _P, _P, _P]),
    "futx_pack_codes_host": (_I32, [_D, _I32, _P, _P, _P, _P]),
    "futx_unpack_weights": (_I32, [_D, _I32, _P, _P, _P, _P, _P]),
    "futx_kv_cache_sizes": (_I32, [_D, _I32, _SZ, _SZ]),
    "futx_kv_append": (_I32, [_D, _I32, _P, _P, _P, _P, ctypes.c_uint32, ctypes.POINTER(futx_kv_cache), _P]),
    "futx_decode_workspace_size": (_I32, [_D, _I32, _I32, _SZ]),
    "futx_decode_block": (_I32, [_D, ctypes.POINTER(futx_block_weights), _I32, _P, _P, _P, _I32, _I32,
                                 ctypes.POINTER(futx_kv_cache), _P, ctypes.c_size_t, _P]),
    "futx_decode_block_noalloc": (_I32, [_D, ctypes.POINTER(futx_block_weights), _I32, _P, _P, _P, _I32, _I32,
                                         ctypes.POINTER(futx_kv_cache), _P]),
    "futx_decode_block_stage": (_I32, [_D, ctypes.POINTER(futx_block_weights), _I32, _P, _P, _P, _I32, _I32,
                                       ctypes.POINTER(futx_kv_cache), _P, ctypes.c_size_t, _I32, _P]),
    "futx_int4_linear": (_I32, [_D, _I32, ctypes.POINTER(futx_qweight), _I32, _P, _P, _P, ctypes.c_size_t, _P]),
    "futx_decode_attention": (_I32, [_D, _I32, _P, _P, _P, _I32, _I32, ctypes.POINTER(futx_kv_cache), _P, _P,
                                     ctypes.c_size_t, _P]),
    "futx_embed": (_I32, [_I32, _I32, _P, _P, _I32, _P, _P]),
    "futx_lm_head": (_I32, [_D, _I32, _P, _I32, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "futx_lm_head_workspace_size": (_I32, [_D, _I32, _I32, _SZ]),
    "futx_fold_head": (_I32, [_I32, _I32, _P, _P, _P]),
    "futx_stream_read": (_I32, [_P, ctypes.c_size_t, _P, _I32, _P]),
    "futx_fp8_packed_sizes": (_I32, [_D, _I32, _SZ, _SZ]),
    "futx_pack_fp8_weights": (_I32, [_D, _I32, _P, _P, _P, _P, _P]),
    "futx_pack_fp8_weights_host": (_I32, [_D, _I32, _P, _P, _P, _P]),
    "futx_fp8_linear_workspace_size": (_I32, [_D, _I32, _I32, _SZ]),
    "futx_fp8_quantize_act": (_I32, [_I32, _I32, _P, _P, _P, _P]),
    "futx_fp8_linear": (_I32, [_D, _I32, ctypes.POINTER(futx_qweight), _I32, _P, _P, _P, ctypes.c_size_t, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


def _check(name, status):
    if status != FUTX_OK:
        raise FutxError(name, status, _lib.futx_last_error().decode(errors="replace"))


def _ptr(x):
    """Pointer of a torch tensor, numpy array, raw int address or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("numpy buffers must be C-contiguous")
        return x.ctypes.data
    if hasattr(x, "data_ptr"):
        if not x.is_contiguous():
            raise ValueError("tensors must be contiguous")
        return x.data_ptr()
    raise TypeError(f"cannot take the address of {type(x)!r}")


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_dims(d):
    """futx_dims from any object with the same attribute names."""
    return futx_dims(d.hidden, d.n_heads, d.n_kv_heads, d.head_dim, d.intermediate, d.w_group,
                     d.had_block, getattr(d, "page_size", 64), d.rms_eps, d.rope_theta)


def _proj(p):
    return PROJ_BY_NAME[p] if isinstance(p, str) else int(p)


def futx_last_error():
    return _lib.futx_last_error().decode(errors="replace")


def futx_packed_sizes(dims, proj):
    pb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check("futx_packed_sizes", _lib.futx_packed_sizes(ctypes.byref(make_dims(dims)), _proj(proj),
                                                       ctypes.byref(pb), ctypes.byref(sb)))
    return pb.value, sb.value


def futx_pack_weights(dims, proj, w_host, gain_host, packed_dev, scales_dev, stream=None):
    w_host = np.ascontiguousarray(w_host, dtype=np.float32)
    g = None if gain_host is None else np.ascontiguousarray(gain_host, dtype=np.float32)
    _check("futx_pack_weights", _lib.futx_pack_weights(ctypes.byref(make_dims(dims)), _proj(proj), _ptr(w_host),
                                                       _ptr(g), _ptr(packed_dev), _ptr(scales_dev),
                                                       _stream(stream)))


def futx_pack_weights_host(dims, proj, w_host, gain_host, packed_host, scales_host):
    w_host = np.ascontiguousarray(w_host, dtype=np.float32)
    g = None if gain_host is None else np.ascontiguousarray(gain_host, dtype=np.float32)
    _check("futx_pack_weights_host", _lib.futx_pack_weights_host(ctypes.byref(make_dims(dims)), _proj(proj),
                                                                 _ptr(w_host), _ptr(g), _ptr(packed_host),
                                                                 _ptr(scales_host)))


def futx_pack_codes(dims, proj, codes_host, scales_host, packed_dev, scales_dev, stream=None):
    codes_host = np.ascontiguousarray(codes_host, dtype=np.uint8)
    scales_host = np.ascontiguousarray(scales_host, dtype=np.uint16)
    _check("futx_pack_codes", _lib.futx_pack_codes(ctypes.byref(make_dims(dims)), _proj(proj), _ptr(codes_host),
                                                   _ptr(scales_host), _ptr(packed_dev), _ptr(scales_dev),
                                                   _stream(stream)))


def futx_pack_codes_host(dims, proj, codes_host, scales_host, packed_host, packed_scales_host):
    codes_host = np.ascontiguousarray(codes_host, dtype=np.uint8)
    scales_host = np.ascontiguousarray(scales_host, dtype=np.uint16)
    _check("futx_pack_codes_host", _lib.futx_pack_codes_host(ctypes.byref(make_dims(dims)), _proj(proj),
                                                             _ptr(codes_host), _ptr(scales_host),
                                                             _ptr(packed_host), _ptr(packed_scales_host)))


def futx_unpack_weights(dims, proj, packed_dev, scales_dev, canon_bytes_host, canon_scales_host, stream=None):
    _check("futx_unpack_weights", _lib.futx_unpack_weights(ctypes.byref(make_dims(dims)), _proj(proj),
                                                           _ptr(packed_dev), _ptr(scales_dev),
                                                           _ptr(canon_bytes_host), _ptr(canon_scales_host),
                                                           _stream(stream)))


def futx_kv_cache_sizes(dims, num_pages):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check("futx_kv_cache_sizes", _lib.futx_kv_cache_sizes(ctypes.byref(make_dims(dims)), int(num_pages),
                                                           ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def make_cache(k_codes, v_codes, k_scales, v_scales, num_pages):
    return futx_kv_cache(_ptr(k_codes), _ptr(v_codes), _ptr(k_scales), _ptr(v_scales), int(num_pages))


def futx_kv_append(dims, n_tokens, k, v, positions, slots, flags, cache, stream=None):
    _check("futx_kv_append", _lib.futx_kv_append(ctypes.byref(make_dims(dims)), int(n_tokens), _ptr(k), _ptr(v),
                                                 _ptr(positions), _ptr(slots), int(flags), ctypes.byref(cache),
                                                 _stream(stream)))


def futx_decode_workspace_size(dims, max_batch, max_context):
    b = ctypes.c_size_t()
    _check("futx_decode_workspace_size", _lib.futx_decode_workspace_size(ctypes.byref(make_dims(dims)),
                                                                         int(max_batch), int(max_context),
                                                                         ctypes.byref(b)))
    return b.value


def make_block_weights(qkv, o, gateup, down):
    """Each argument is a (packed, scales) pair of device buffers."""
    return futx_block_weights(*(futx_qweight(_ptr(p), _ptr(s)) for p, s in (qkv, o, gateup, down)))


def futx_decode_block(dims, weights, batch, x, cached_lens, block_table, max_pages_per_seq, max_context,
                      cache, workspace, workspace_bytes, stream=None):
    _check("futx_decode_block", _lib.futx_decode_block(ctypes.byref(make_dims(dims)), ctypes.byref(weights),
                                                       int(batch), _ptr(x), _ptr(cached_lens), _ptr(block_table),
                                                       int(max_pages_per_seq), int(max_context),
                                                       ctypes.byref(cache), _ptr(workspace), int(workspace_bytes),
                                                       _stream(stream)))


def futx_decode_block_noalloc(dims, weights, batch, x, cached_lens, block_table, max_pages_per_seq, max_context,
                              cache, stream=None):
    _check("futx_decode_block_noalloc",
           _lib.futx_decode_block_noalloc(ctypes.byref(make_dims(dims)), ctypes.byref(weights), int(batch), _ptr(x),
                                          _ptr(cached_lens), _ptr(block_table), int(max_pages_per_seq),
                                          int(max_context), ctypes.byref(cache), _stream(stream)))


def futx_decode_block_stage(dims, weights, batch, x, cached_lens, block_table, max_pages_per_seq, max_context,
                            cache, workspace, workspace_bytes, stage, stream=None):
    _check("futx_decode_block_stage",
           _lib.futx_decode_block_stage(ctypes.byref(make_dims(dims)), ctypes.byref(weights), int(batch), _ptr(x),
                                        _ptr(cached_lens), _ptr(block_table), int(max_pages_per_seq),
                                        int(max_context), ctypes.byref(cache), _ptr(workspace),
                                        int(workspace_bytes), int(stage), _stream(stream)))


def futx_int4_linear(dims, proj, qweight, batch, act, out, workspace, workspace_bytes, stream=None):
    qw = futx_qweight(_ptr(qweight[0]), _ptr(qweight[1])) if isinstance(qweight, tuple) else qweight
    _check("futx_int4_linear", _lib.futx_int4_linear(ctypes.byref(make_dims(dims)), _proj(proj), ctypes.byref(qw),
                                                     int(batch), _ptr(act), _ptr(out), _ptr(workspace),
                                                     int(workspace_bytes), _stream(stream)))


def futx_decode_attention(dims, batch, qkv, cached_lens, block_table, max_pages_per_seq, max_context, cache, out,
                          workspace, workspace_bytes, stream=None):
    _check("futx_decode_attention", _lib.futx_decode_attention(ctypes.byref(make_dims(dims)), int(batch),
                                                               _ptr(qkv), _ptr(cached_lens), _ptr(block_table),
                                                               int(max_pages_per_seq), int(max_context),
                                                               ctypes.byref(cache), _ptr(out), _ptr(workspace),
                                                               int(workspace_bytes), _stream(stream)))


def futx_embed(hidden, vocab, table_bf16, tokens, batch, x, stream=None):
    _check("futx_embed", _lib.futx_embed(int(hidden), int(vocab), _ptr(table_bf16), _ptr(tokens), int(batch),
                                         _ptr(x), _stream(stream)))


def futx_lm_head_workspace_size(dims, vocab, max_batch):
    b = ctypes.c_size_t()
    _check("futx_lm_head_workspace_size",
           _lib.futx_lm_head_workspace_size(ctypes.byref(make_dims(dims)), int(vocab), int(max_batch),
                                            ctypes.byref(b)))
    return b.value


def futx_lm_head(dims, vocab, w_bf16, batch, x, logits, top1, workspace, workspace_bytes, stream=None):
    _check("futx_lm_head", _lib.futx_lm_head(ctypes.byref(make_dims(dims)), int(vocab), _ptr(w_bf16), int(batch),
                                             _ptr(x), _ptr(logits), _ptr(top1), _ptr(workspace),
                                             int(workspace_bytes), _stream(stream)))


def futx_fold_head(vocab, hidden, w_bf16_host, gain_host, out_bf16_host):
    gain = np.ascontiguousarray(gain_host, np.float32)  # kept alive across the call
    _check("futx_fold_head", _lib.futx_fold_head(int(vocab), int(hidden), _ptr(w_bf16_host), _ptr(gain),
                                                 _ptr(out_bf16_host)))


def futx_stream_read(buf, nbytes, sink, workgroups, stream=None):
    _check("futx_stream_read", _lib.futx_stream_read(_ptr(buf), int(nbytes), _ptr(sink), int(workgroups),
                                                     _stream(stream)))


def futx_fp8_packed_sizes(dims, proj):
    pb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check("futx_fp8_packed_sizes", _lib.futx_fp8_packed_sizes(ctypes.byref(make_dims(dims)), _proj(proj),
                                                               ctypes.byref(pb), ctypes.byref(sb)))
    return pb.value, sb.value


def futx_pack_fp8_weights(dims, proj, w_host, gain_host, packed_dev, scales_dev, stream=None):
    w_host = np.ascontiguousarray(w_host, dtype=np.float32)
    g = None if gain_host is None else np.ascontiguousarray(gain_host, dtype=np.float32)
    _check("futx_pack_fp8_weights", _lib.futx_pack_fp8_weights(ctypes.byref(make_dims(dims)), _proj(proj),
                                                               _ptr(w_host), _ptr(g), _ptr(packed_dev),
                                                               _ptr(scales_dev), _stream(stream)))


def futx_pack_fp8_weights_host(dims, proj, w_host, gain_host, packed_host, scales_host):
    w_host = np.ascontiguousarray(w_host, dtype=np.float32)
    g = None if gain_host is None else np.ascontiguousarray(gain_host, dtype=np.float32)
    _check("futx_pack_fp8_weights_host", _lib.futx_pack_fp8_weights_host(ctypes.byref(make_dims(dims)), _proj(proj),
                                                                         _ptr(w_host), _ptr(g), _ptr(packed_host),
                                                                         _ptr(scales_host)))


def futx_fp8_linear_workspace_size(dims, proj, max_batch):
    b = ctypes.c_size_t()
    _check("futx_fp8_linear_workspace_size",
           _lib.futx_fp8_linear_workspace_size(ctypes.byref(make_dims(dims)), _proj(proj), int(max_batch),
                                               ctypes.byref(b)))
    return b.value


def futx_fp8_quantize_act(k, rows, act, codes, scales, stream=None):
    _check("futx_fp8_quantize_act", _lib.futx_fp8_quantize_act(int(k), int(rows), _ptr(act), _ptr(codes),
                                                               _ptr(scales), _stream(stream)))


def futx_fp8_linear(dims, proj, qweight, batch, act, out, workspace, workspace_bytes, stream=None):
    qw = futx_qweight(_ptr(qweight[0]), _ptr(qweight[1])) if isinstance(qweight, tuple) else qweight
    _check("futx_fp8_linear", _lib.futx_fp8_linear(ctypes.byref(make_dims(dims)), _proj(proj), ctypes.byref(qw),
                                                   int(batch), _ptr(act), _ptr(out), _ptr(workspace),
                                                   int(workspace_bytes), _stream(stream)))
