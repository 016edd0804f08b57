"""Decode attention over the rotated INT4 cache (oracle, test infrastructure only).

What the pages fix: decode reads the whole KV cache each step and is bound by
that read [kongchang.com/en, "Why do Prefill and Decode need different
quantization strategies?", KV-cache explainer]; decode attention uses an INT4
KV-cache copy rotated by a block-diagonal Hadamard transform [ABS]; the
rotation is undone after use [INT4, Hadamard explainer paragraph].

Readings: scaled dot-product attention with scale 1/sqrt(d); grouped-query
attention, query head i reads KV head floor(i / G) with G = n_heads /
n_kv_heads; no mask besides the length; the new token is written to the cache
first and read back quantized like every cached token.  Queries and keys are
both rotated by the same block Hadamard, so scores equal those of unrotated
vectors (orthogonality); the weighted sum of rotated values is rotated back
by the same (self-inverse) matrix.

``decode_attention``       fp64, vectorized, max-subtracted softmax.
``attention_bruteforce_loops``  the same definition in plain Python loops
                           (tiny inputs only), an independent pin.
``attention_chunked``      splits the token range at arbitrary points and
                           merges (max, sum, accumulator) partials; equals the
                           unsplit result to 1e-12 (pinned).
"""

import math

import numpy as np

from .hadamard import block_diag_rotate


def decode_attention(q_rot, k_hat, v_hat, hb):
    """Attention output for one sequence.

    q_rot  [nq][d]          rotated query (fp64)
    k_hat  [T][nkv][d]      dequantized rotated keys, T = cached + 1
    v_hat  [T][nkv][d]      dequantized rotated values
    returns o [nq][d]       = BD_H(softmax(q k^T / sqrt d) v), fp64
    """
    q_rot = np.asarray(q_rot, np.float64)
    k_hat = np.asarray(k_hat, np.float64)
    v_hat = np.asarray(v_hat, np.float64)
    nq, d = q_rot.shape
    nkv = k_hat.shape[1]
    g = nq // nkv
    out = np.empty((nq, d))
    for i in range(nq):
        h = i // g
        z = k_hat[:, h, :] @ q_rot[i] / math.sqrt(d)
        p = np.exp(z - z.max())
        p /= p.sum()
        out[i] = p @ v_hat[:, h, :]
    return block_diag_rotate(out, hb)


def attention_bruteforce_loops(q_rot, k_hat, v_hat, hb):
    """The definition written out with Python loops (tiny inputs only)."""
    nq, d = len(q_rot), len(q_rot[0])
    t_len, nkv = len(k_hat), len(k_hat[0])
    g = nq // nkv
    res = []
    for i in range(nq):
        h = i // g
        scores = []
        for t in range(t_len):
            acc = 0.0
            for c in range(d):
                acc += float(q_rot[i][c]) * float(k_hat[t][h][c])
            scores.append(acc / math.sqrt(d))
        mx = max(scores)
        w = [math.exp(s - mx) for s in scores]
        tot = sum(w)
        o = []
        for c in range(d):
            acc = 0.0
            for t in range(t_len):
                acc += w[t] * float(v_hat[t][h][c])
            o.append(acc / tot)
        res.append(o)
    # inverse rotation, block by block, as explicit sums
    from .hadamard import sylvester

    hmat = sylvester(hb)
    out = []
    for o in res:
        r = []
        for c in range(d):
            blk, j = divmod(c, hb)
            acc = 0.0
            for m in range(hb):
                acc += float(hmat[j][m]) * o[blk * hb + m]
            r.append(acc / math.sqrt(hb))
        out.append(r)
    return np.array(out)


def _partial(qv, k_h, v_h):
    """(m, l, acc) of one chunk for one query vector."""
    d = qv.shape[0]
    z = k_h @ qv / math.sqrt(d)
    m = z.max()
    p = np.exp(z - m)
    return m, p.sum(), p @ v_h


def softmax_merge(parts):
    """Merge chunk partials (m_c, l_c, acc_c): m = max m_c,
    l = sum e^(m_c - m) l_c, acc = sum e^(m_c - m) acc_c; returns acc / l."""
    m = max(p[0] for p in parts)
    l_tot = sum(math.exp(p[0] - m) * p[1] for p in parts)
    acc = sum(math.exp(p[0] - m) * p[2] for p in parts)
    return acc / l_tot


def attention_chunked(q_rot, k_hat, v_hat, hb, bounds):
    """Same as ``decode_attention`` but over token chunks [bounds[j], bounds[j+1])."""
    q_rot = np.asarray(q_rot, np.float64)
    k_hat = np.asarray(k_hat, np.float64)
    v_hat = np.asarray(v_hat, np.float64)
    nq, d = q_rot.shape
    nkv = k_hat.shape[1]
    g = nq // nkv
    out = np.empty((nq, d))
    for i in range(nq):
        h = i // g
        parts = [
            _partial(q_rot[i], k_hat[a:b, h, :], v_hat[a:b, h, :])
            for a, b in zip(bounds[:-1], bounds[1:])
            if b > a
        ]
        out[i] = softmax_merge(parts)
    return block_diag_rotate(out, hb)
