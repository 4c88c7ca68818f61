"""Decode attention over a JoLT-compressed cache, and dense decode attention.

TEST INFRASTRUCTURE (see the package docstring).  What this module computes:
the plain definition of one decode step's attention over the cache that the
stored cells decode to (factors plus de-rotated residual).  A fused kernel
that works on the factors directly evaluates the same quantity in another
order, so it must produce the same numbers.  Source: "A JoLT for the KV
cache" (arXiv 2607.12550v4 summary), Abstract and §4.5 (fused decode over
stored factors and packed residuals; key tiles rebuilt because RoPE and the
factorisation do not commute).  Written out:

  K^[l, h] = A_K G_K[l', h] B_K^T + [b_K > 0] deq(codes_K[l', h]) Pi^T  (V^ alike)
  s_t      = scale * rope(q_j, q_pos) . rope(K^[l, h]_t, t)
  p        = softmax(s)                (max-subtracted, float64)
  o_j      = sum_t p_t V^[l, h]_t

for query head j served by KV head h = floor(j / H_grp) (grouped-query
attention: the sarnas.ru post's 70B example, 8 query heads per KV head), layer
l in group g at index l' = l - group_start[g].  Readings taken: the query sits
at position q_pos (normally T) and attends only to the T cached tokens; the
output is float32-sized but computed here in float64.
"""
import numpy as np

from .quant import dequantize, unpack
from .rope import rope
from .rotation import rotation


def group_of(cache, layer):
    gsl = cache["group_start"]
    for g in range(len(gsl) - 1):
        if gsl[g] <= layer < gsl[g + 1]:
            return g, layer - gsl[g]
    raise IndexError(layer)


def residual(cell, lp, d, heads=None):
    """deq(codes) in the rotated basis for layer index lp: [H, T, d] (or the
    listed heads only) or None."""
    if cell["bits"] == 0:
        return None
    hs = slice(None) if heads is None else list(heads)
    codes = unpack(cell["codes"][lp][hs], cell["bits"], d)
    return dequantize(codes, cell["scales"][lp][hs], cell["bits"])


def decode_cell(cell, lp, d, Pi, heads=None):
    """X^[lp] of one stored cell: [H, T, d] float64 (or [len(heads), T, d]
    for the listed heads; large workloads decode a sample of heads)."""
    hs = slice(None) if heads is None else list(heads)
    A = cell["A"].astype(np.float64)
    B = cell["B"].astype(np.float64)
    G = cell["G"][lp][hs].astype(np.float64)
    H = G.shape[0]
    T = A.shape[0]
    out = np.zeros((H, T, d))
    if cell["r_T"] > 0:
        out += np.einsum("tr,hrs,fs->htf", A, G, B, optimize=True)
    R = residual(cell, lp, d, heads)
    if R is not None:
        out += R @ Pi.T
    return out


def softmax_attention(qr, Kr, V, scale):
    """qr [Hg, d], Kr [T, d], V [T, d] -> [Hg, d] (float64)."""
    s = scale * (qr @ Kr.T)
    s = s - np.max(s, axis=-1, keepdims=True)
    p = np.exp(s)
    p /= np.sum(p, axis=-1, keepdims=True)
    return p @ V


def decode_layer(cache, layer, q, q_pos, inv_freq, scale, Pi=None, heads=None):
    """One sequence, one layer: q [H_q, d] -> o [H_q, d] (rows of ``heads`` only
    when a subset of KV heads is requested; other rows are NaN)."""
    d, H, H_q, T = cache["d"], cache["H"], cache["H_q"], cache["T"]
    if Pi is None:
        Pi = rotation(cache["rotation_seed"], d)
    g, lp = group_of(cache, layer)
    cK, cV = cache["cells"][g]
    Hg = H_q // H
    heads = range(H) if heads is None else heads
    qr = rope(np.asarray(q, dtype=np.float64), q_pos, inv_freq)
    pos = np.arange(T)
    out = np.full((H_q, d), np.nan)
    heads = list(heads)
    Khat = decode_cell(cK, lp, d, Pi, heads)
    Vhat = decode_cell(cV, lp, d, Pi, heads)
    for n, h in enumerate(heads):
        Kr = rope(Khat[n], pos, inv_freq)
        out[h * Hg:(h + 1) * Hg] = softmax_attention(qr[h * Hg:(h + 1) * Hg], Kr, Vhat[n], scale)
    return out


def decode_layer_tail(cache, layer, q, q_pos, inv_freq, scale, k_tail, v_tail, Pi=None):
    """One sequence, one layer, with an uncompressed tail: the query attends
    to the T compressed tokens (decoded, keys rotated to positions 0..T-1)
    followed by the tail's n tokens, whose keys k_tail [H, n, d] are given
    already rotated to their positions, and values v_tail [H, n, d].  One
    softmax over all T + n tokens.  (A decode loop appends each generated
    token's key and value to such a tail until the next compression; the
    JoLT summary's §5 notes that its prefill compressor alone does not
    cover streaming generation.)"""
    d, H, H_q, T = cache["d"], cache["H"], cache["H_q"], cache["T"]
    if Pi is None:
        Pi = rotation(cache["rotation_seed"], d)
    g, lp = group_of(cache, layer)
    cK, cV = cache["cells"][g]
    Hg = H_q // H
    qr = rope(np.asarray(q, dtype=np.float64), q_pos, inv_freq)
    Khat = decode_cell(cK, lp, d, Pi)
    Vhat = decode_cell(cV, lp, d, Pi)
    out = np.empty((H_q, d))
    for h in range(H):
        Kr = np.concatenate([rope(Khat[h], np.arange(T), inv_freq),
                             np.asarray(k_tail[h], dtype=np.float64)])
        V = np.concatenate([Vhat[h], np.asarray(v_tail[h], dtype=np.float64)])
        out[h * Hg:(h + 1) * Hg] = softmax_attention(qr[h * Hg:(h + 1) * Hg], Kr, V, scale)
    return out


def decode_attention(caches, layer, q, q_pos, inv_freq, scale):
    """Batch of sequences: q [B, H_q, d], q_pos [B] -> [B, H_q, d]."""
    Pi_cache = {}
    out = []
    for b, c in enumerate(caches):
        key = (c["rotation_seed"], c["d"])
        if key not in Pi_cache:
            Pi_cache[key] = rotation(*key)
        out.append(decode_layer(c, layer, q[b], int(q_pos[b]), inv_freq, scale, Pi_cache[key]))
    return np.stack(out)


def factored_value_output(p, cellV, lp, h, d, Pi):
    """The value path by linearity, never forming V^:
    o = (p A_V) G_V[lp, h] B_V^T + (p deq_V[lp, h]) Pi^T  for p [Hg, T]."""
    A = cellV["A"].astype(np.float64)
    o = np.zeros((p.shape[0], d))
    if cellV["r_T"] > 0:
        a = p @ A
        o += (a @ cellV["G"][lp, h].astype(np.float64)) @ cellV["B"].astype(np.float64).T
    R = residual(cellV, lp, d)
    if R is not None:
        o += (p @ R[h]) @ Pi.T
    return o


def dense_attention(k_rope, v, q, q_pos, inv_freq, scale):
    """Dense decode over post-RoPE keys: k_rope, v [B, H, T, d]; q [B, H_q, d]
    (pre-RoPE; rotated to q_pos here) -> [B, H_q, d]."""
    Bn, H, T, d = k_rope.shape
    H_q = q.shape[1]
    Hg = H_q // H
    out = np.empty((Bn, H_q, d))
    for b in range(Bn):
        qr = rope(np.asarray(q[b], dtype=np.float64), int(q_pos[b]), inv_freq)
        for h in range(H):
            out[b, h * Hg:(h + 1) * Hg] = softmax_attention(
                qr[h * Hg:(h + 1) * Hg], np.asarray(k_rope[b, h], dtype=np.float64),
                np.asarray(v[b, h], dtype=np.float64), scale)
    return out
