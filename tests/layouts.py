"""Test-side decoders of the device layouts (written from the layout
description, independent of the library and of the oracle).

Weights: packed[nt][kb][L][16 bytes]; word s (bytes 4s..4s+3, little endian)
of lane L holds row nt*16 + L%16, inputs kb*128 + 32 s + 8 (L // 16) + e;
element e is stored as code + 8 in bits 3..6 of the word rotated left by
4 (e // 2) + 16 (e % 2).  GATEUP physical tile 2t = gate rows 16t..,
2t+1 = up rows 16t..  Scales: see decode_scales.

KV cache per (page, KV head): keys [tt][L][D/8 bytes] with token tt*16 + L%16
and word s = channels 32 s + 8 (L//16) + e; values [tb][cg][L][16 bytes] with
word c4 = channel cg*64 + 16 c4 + L%16 and element e = token tb*32 + tok(L//16, e),
tok(g, e) = 4g + e (e < 4) else 16 + 4g + e - 4.
"""

import numpy as np


def _nibbles(words):
    """uint32 [...] -> codes int8 [..., 8] in element order e = 0..7."""
    w = np.asarray(words, np.uint32)
    out = np.empty(w.shape + (8,), np.int8)
    for e in range(8):
        r = 4 * (e // 2) + 16 * (e % 2)
        rot = (w >> np.uint32(r)) | (w << np.uint32(32 - r)) if r else w
        out[..., e] = ((rot >> np.uint32(3)) & np.uint32(15)).astype(np.int8) - 8
    return out


def decode_weights(packed, n, k):
    """Device-order bytes of an [n][k] projection -> codes int8 [n_phys][k]."""
    b = np.asarray(packed, np.uint8).reshape(n // 16, k // 128, 4, 16, 4, 4)  # nt kb g i s byte
    words = b.copy().view(np.uint32)[..., 0]  # nt kb g i s
    codes = _nibbles(words)  # nt kb g i s e
    codes = codes.transpose(0, 3, 1, 4, 2, 5)  # nt i kb s g e
    return codes.reshape(n, k)


def decode_scales(scales, n, k, group):
    """Device-order fp16 group scales of an [n][k] projection -> [n_phys][k // group].

    Blocked per 16-row tile and 8 K blocks of 128: [nt][kb // 8][i][slot], slot
    = (kb % 8) * (128 // group) + (g % (128 // group)); the last block of 8 is
    padded when k / 128 is not a multiple of 8."""
    per_kb = 128 // group
    kb8 = (k // 128 + 7) // 8
    s = np.asarray(scales).view(np.uint16).reshape(n // 16, kb8, 16, 8 * per_kb)
    s = s.transpose(0, 2, 1, 3).reshape(n, kb8 * 8 * per_kb)
    return s[:, : k // group].view(np.float16)


def gateup_logical_order(phys, inter):
    """Rows of a GATEUP matrix in physical order -> logical order (gate rows then up rows)."""
    p = np.asarray(phys)
    n = p.shape[0]
    rows = np.arange(n)
    tile, i = rows // 16, rows % 16
    logical = (tile % 2) * inter + (tile // 2) * 16 + i
    out = np.empty_like(p)
    out[logical] = p
    return out


def decode_k_page(kbytes, d):
    """Key codes of one (page, head): bytes [64 * d / 2] -> codes int8 [64][d]."""
    b = np.asarray(kbytes, np.uint8).reshape(4, 4, 16, d // 32, 4)  # tt g i s byte
    words = b.copy().view(np.uint32)[..., 0]  # tt g i s
    codes = _nibbles(words)  # tt g i s e
    codes = codes.transpose(0, 2, 3, 1, 4)  # tt i s g e
    return codes.reshape(64, d)


def decode_v_page(vbytes, d):
    """Value codes of one (page, head): bytes [64 * d / 2] -> codes int8 [64][d]."""
    b = np.asarray(vbytes, np.uint8).reshape(2, d // 64, 4, 16, 4, 4)  # tb cg g i c4 byte
    words = b.copy().view(np.uint32)[..., 0]  # tb cg g i c4
    codes = _nibbles(words)  # tb cg g i c4 e
    out = np.empty((64, d), np.int8)
    for tb in range(2):
        for g in range(4):
            for e in range(8):
                t = tb * 32 + (4 * g + e if e < 4 else 16 + 4 * g + e - 4)
                for cg in range(d // 64):
                    for c4 in range(4):
                        ch = cg * 64 + 16 * c4 + np.arange(16)
                        out[t, ch] = codes[tb, cg, g, :, c4, e]
    return out


def decode_cache(k_codes, v_codes, k_scales, v_scales, num_pages, nkv, d):
    """Whole cache -> (k codes [pages][nkv][64][d], k scales fp16 [pages][nkv][64], v codes, v scales).

    The same index maps as decode_k_page / decode_v_page, over all pages and
    heads at once: key token tt*16 + i, channel 32 s + 8 g + e; value token
    tb*32 + 16 h + 4 g + e4 (element e = 4 h + e4), channel cg*64 + 16 c4 + i."""
    P = num_pages
    kb = np.asarray(k_codes, np.uint8).reshape(P, nkv, 4, 4, 16, d // 32, 4)  # tt g i s byte
    kw = kb.copy().view(np.uint32)[..., 0]
    K = _nibbles(kw)  # P h tt g i s e
    K = K.transpose(0, 1, 2, 4, 5, 3, 6).reshape(P, nkv, 64, d)  # P h tt i s g e
    vb = np.asarray(v_codes, np.uint8).reshape(P, nkv, 2, d // 64, 4, 16, 4, 4)  # tb cg g i c4 byte
    vw = vb.copy().view(np.uint32)[..., 0]
    V = _nibbles(vw).reshape(P, nkv, 2, d // 64, 4, 16, 4, 2, 4)  # P h tb cg g i c4 hh e4
    V = V.transpose(0, 1, 2, 7, 4, 8, 3, 6, 5).reshape(P, nkv, 64, d)  # P h tb hh g e4 cg c4 i
    ks = np.asarray(k_scales).view(np.float16).reshape(P, nkv, 64)
    vs = np.asarray(v_scales).view(np.float16).reshape(P, nkv, 64)
    return K, ks, V, vs


def decode_fp8_weights(packed, scales, n, k):
    """FP8 device order of an [n][k] projection -> (codes uint8 [n][k], fp32
    scales [n][k // 128]).  Bytes [nt][kb][L][32]: lane L holds row
    nt*16 + L%16, byte 8 s + e holds input kb*128 + 32 s + 8 (L//16) + e;
    scales [nt][kb][16]."""
    b = np.asarray(packed, np.uint8).reshape(n // 16, k // 128, 4, 16, 4, 8)  # nt kb g i s e
    codes = b.transpose(0, 3, 1, 4, 2, 5).reshape(n, k)  # nt i kb s g e
    s = np.asarray(scales).view(np.float32).reshape(n // 16, k // 128, 16).transpose(0, 2, 1).reshape(n, k // 128)
    return codes, s
