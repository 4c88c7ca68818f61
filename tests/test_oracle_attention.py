"""Pins for oracle.rope and oracle.attention.

* RoPE: position 0 is the identity; norm preserving; equals the complex
  formulation (x_i + i x_{i+d/2}) e^{i theta_i}; scores depend on the
  position difference only (to the float32 angle rounding);
* decode attention at full ranks and b = 0 (float64 factors) equals plain
  RoPE attention on the raw cache to 1e-12;
* a brute-force triple loop equals the vectorised decode on tiny inputs;
* q = 0 gives the mean of V^; T = 1 gives V^_0; GQA with one query per KV
  head equals MHA run head by head;
* the factored value path (p A_V) G_V B_V^T + (p deq_V) Pi^T equals p V^;
* dense decode over rope(K^), V^ equals the compressed decode;
* compressed decode with a residual is closer to raw attention than
  without it (the residual is added, with the right sign and rotation).
"""
import math

import numpy as np
import pytest

from oracle import attention as att
from oracle.compress import compress
from oracle.quant import dequantize, unpack
from oracle.rope import angles, rope
from oracle.rotation import rotation
from workloads import gen

INV64 = gen.rope_inv_freq_input(1e4, 64)


def test_rope_identity_at_zero_and_norm():
    x = np.random.default_rng(0).standard_normal((5, 64))
    assert np.array_equal(rope(x, 0, INV64), x)
    y = rope(x, 12345, INV64)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)


def test_rope_complex_form():
    x = np.random.default_rng(1).standard_normal(64)
    t = 777
    a = angles(t, INV64).astype(np.float64)
    z = (x[:32] + 1j * x[32:]) * np.exp(1j * a)
    assert np.allclose(rope(x, t, INV64), np.concatenate([z.real, z.imag]), atol=1e-14)


def test_rope_relative_position():
    g = np.random.default_rng(2)
    q, k = g.standard_normal(64), g.standard_normal(64)
    s = [rope(q, m, INV64) @ rope(k, m - 5, INV64) for m in (5, 50, 500)]
    assert np.allclose(s, s[0], atol=1e-4)


def rand_groups(seed, gs, H, T, d):
    return [(gen.kv_tensor((97, seed, g, 0), gs, H, T, d, 1.0, True, 2),
             gen.kv_tensor((97, seed, g, 1), gs, H, T, d, 0.3, False, 0)) for g in range(2)]


def test_full_rank_no_residual_is_raw_attention():
    gs, H, H_q, T, d = 2, 2, 4, 48, 16
    groups = rand_groups(0, gs, H, T, d)
    full = (min(T, gs * H * d), d, 0)
    cache = compress(groups, [(full, full)] * 2, "f64", 5, H_q, [0, 2, 4])
    q = np.random.default_rng(1).standard_normal((H_q, d))
    inv = gen.rope_inv_freq_input(1e4, d)
    for layer in range(4):
        o = att.decode_layer(cache, layer, q, T, inv, 0.25)
        XK, XV = groups[layer // 2]
        for h in range(H):
            Kr = rope(XK[layer % 2, h], np.arange(T), inv)
            want = att.softmax_attention(rope(q[2 * h:2 * h + 2], T, inv), Kr, XV[layer % 2, h], 0.25)
            assert np.max(np.abs(o[2 * h:2 * h + 2] - want)) < 1e-12


def tiny_cache(bits=(4, 2), seed=0, T=12, d=8, H=2, H_q=4):
    groups = rand_groups(seed, 1, H, T, d)[:1]
    return compress(groups, [((8, 4, bits[0]), (4, 8, bits[1]))], "bf16", 9, H_q, [0, 1]), groups


def test_brute_force_loop():
    cache, _ = tiny_cache()
    d, T, H, H_q = 8, 12, 2, 4
    inv = gen.rope_inv_freq_input(5e5, d)
    q = np.random.default_rng(3).standard_normal((H_q, d))
    o = att.decode_layer(cache, 0, q, 40, inv, 0.3)
    Pi = rotation(9, d)
    cK, cV = cache["cells"][0]
    def elem(cell, h, t, f):
        v = sum(float(cell["A"][t, r]) * float(cell["G"][0, h, r, s]) * float(cell["B"][f, s])
                for r in range(cell["r_T"]) for s in range(cell["r_F"]))
        if cell["bits"]:
            L = (1 << cell["bits"]) - 1
            codes = unpack(cell["codes"][0, h, t], cell["bits"], d)
            v += sum((int(codes[i]) - L / 2) * float(cell["scales"][0, h, t]) * float(Pi[f, i])
                     for i in range(d))
        return v
    for j in range(H_q):
        h = j // 2
        a_q = angles(40, inv).astype(np.float64)
        qr = [q[j, i] * math.cos(a_q[i % 4]) + (-q[j, i + 4] if i < 4 else q[j, i - 4]) * math.sin(a_q[i % 4]) for i in range(d)]
        s = []
        for t in range(T):
            k = [elem(cK, h, t, f) for f in range(d)]
            a_k = angles(t, inv).astype(np.float64)
            kr = [k[i] * math.cos(a_k[i % 4]) + (-k[i + 4] if i < 4 else k[i - 4]) * math.sin(a_k[i % 4]) for i in range(d)]
            s.append(0.3 * sum(qr[i] * kr[i] for i in range(d)))
        m = max(s)
        p = [math.exp(x - m) for x in s]
        Z = sum(p)
        for f in range(d):
            want = sum(p[t] / Z * elem(cV, h, t, f) for t in range(T))
            assert abs(o[j, f] - want) < 1e-12


def test_q_zero_gives_mean_and_T1_gives_first():
    cache, _ = tiny_cache()
    inv = gen.rope_inv_freq_input(1e4, 8)
    o = att.decode_layer(cache, 0, np.zeros((4, 8)), 12, inv, 1.0)
    V = att.decode_cell(cache["cells"][0][1], 0, 8, rotation(9, 8))
    for j in range(4):
        assert np.allclose(o[j], V[j // 2].mean(axis=0), atol=1e-13)
    c1 = {k: v for k, v in cache.items()}
    c1["T"] = 1
    c1["cells"] = [tuple(dict(c, A=c["A"][:1], codes=c["codes"][:, :, :1], scales=c["scales"][:, :, :1])
                         for c in cache["cells"][0])]
    o1 = att.decode_layer(c1, 0, np.random.default_rng(0).standard_normal((4, 8)), 1, inv, 1.0)
    for j in range(4):
        assert np.allclose(o1[j], V[j // 2, 0], atol=1e-13)


def test_head_subset_matches_full_decode():
    """Decoding a sample of KV heads gives exactly those rows of the full
    decode (the large GPU parity cases sample heads this way)."""
    cache = gen.small_cache(11, 50, 4, 8, 16, [((8, 8, 4), (8, 8, 2))], [2], factor_dtype="f32")
    inv = gen.rope_inv_freq_input(1e4, 16)
    q = np.random.default_rng(3).standard_normal((8, 16))
    full = att.decode_layer(cache, 1, q, 50, inv, 0.25)
    sub = att.decode_layer(cache, 1, q, 50, inv, 0.25, heads=[3, 1])
    assert np.array_equal(sub[2:4], full[2:4]) and np.array_equal(sub[6:8], full[6:8])
    assert np.isnan(sub[0:2]).all() and np.isnan(sub[4:6]).all()


def test_gqa_equals_mha_head_by_head():
    cache, _ = tiny_cache(H_q=2)          # one query per KV head
    inv = gen.rope_inv_freq_input(1e4, 8)
    q = np.random.default_rng(4).standard_normal((2, 8))
    o = att.decode_layer(cache, 0, q, 12, inv, 0.7)
    Pi = rotation(9, 8)
    K = att.decode_cell(cache["cells"][0][0], 0, 8, Pi)
    V = att.decode_cell(cache["cells"][0][1], 0, 8, Pi)
    for h in range(2):
        want = att.softmax_attention(rope(q[h:h + 1], 12, inv), rope(K[h], np.arange(12), inv), V[h], 0.7)
        assert np.allclose(o[h], want[0], atol=1e-14)


@pytest.mark.parametrize("bits", [(0, 0), (4, 2), (2, 8)])
def test_factored_value_path(bits):
    cache, _ = tiny_cache(bits)
    Pi = rotation(9, 8)
    V = att.decode_cell(cache["cells"][0][1], 0, 8, Pi)
    p = np.random.default_rng(5).random((2, 12))
    for h in range(2):
        assert np.allclose(att.factored_value_output(p, cache["cells"][0][1], 0, h, 8, Pi), p @ V[h],
                           atol=1e-12)


def test_dense_equals_compressed_decode():
    cache, _ = tiny_cache()
    inv = gen.rope_inv_freq_input(1e4, 8)
    Pi = rotation(9, 8)
    K = att.decode_cell(cache["cells"][0][0], 0, 8, Pi)
    V = att.decode_cell(cache["cells"][0][1], 0, 8, Pi)
    Kr = rope(K, np.arange(12), inv)
    q = np.random.default_rng(6).standard_normal((1, 4, 8))
    a = att.dense_attention(Kr[None], V[None], q, [12], inv, 0.5)
    b = att.decode_attention([cache], 0, q, [12], inv, 0.5)
    assert np.allclose(a, b, atol=1e-13)


def test_residual_improves_attention():
    gs, H, H_q, T, d = 1, 2, 4, 64, 32
    groups = rand_groups(7, gs, H, T, d)[:1]
    inv = gen.rope_inv_freq_input(1e4, d)
    q = np.random.default_rng(8).standard_normal((H_q, d))
    XK, XV = groups[0]
    raw = np.concatenate([att.softmax_attention(rope(q[2 * h:2 * h + 2], T, inv),
                                                rope(XK[0, h], np.arange(T), inv), XV[0, h], 0.2)
                          for h in range(H)])
    errs = []
    for b in (0, 4, 8):
        cache = compress(groups, [((8, 8, b), (8, 8, b))], "f32", 1, H_q, [0, 1])
        errs.append(np.linalg.norm(att.decode_layer(cache, 0, q, T, inv, 0.2) - raw))
    assert errs[0] > errs[1] > errs[2]


# ------------------------------------------------------------ dense tail --
def _tail_case(seed, n):
    from oracle.compress import compress
    g = np.random.default_rng(seed)
    T, d, H, H_q = 40, 16, 2, 4
    X = [gen.kv_tensor((94, seed, 0, tau), 1, H, T, d, 1.0 - 0.7 * tau, tau == 0, 1, rank=8)
         for tau in (0, 1)]
    c = compress([tuple(X)], [((16, 8, 4), (16, 8, 2))], "f32", 5, H_q, [0, 1])
    inv = gen.rope_inv_freq_input(1e4, d)
    q = g.standard_normal((H_q, d))
    kt = g.standard_normal((H, n, d))
    vt = g.standard_normal((H, n, d)) * 2
    return c, inv, q, kt, vt


def test_tail_of_length_zero_is_the_compressed_decode():
    c, inv, q, kt, vt = _tail_case(0, 0)
    a = att.decode_layer_tail(c, 0, q, 40, inv, 0.3, kt, vt)
    b = att.decode_layer(c, 0, q, 40, inv, 0.3)
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def test_tail_duplicating_the_prefix_changes_nothing():
    """Attending to every token twice (the tail repeats the decoded, rotated
    prefix) gives the same softmax average."""
    c, inv, q, _, _ = _tail_case(1, 0)
    Pi = rotation(5, 16)
    K = att.decode_cell(c["cells"][0][0], 0, 16, Pi)
    V = att.decode_cell(c["cells"][0][1], 0, 16, Pi)
    kt = np.stack([rope(K[h], np.arange(40), inv) for h in range(2)])
    a = att.decode_layer_tail(c, 0, q, 40, inv, 0.3, kt, V)
    b = att.decode_layer(c, 0, q, 40, inv, 0.3)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_tail_equals_merge_of_two_softmax_partials():
    """The (max, sum) merge of a partial over the prefix and one over the
    tail is the softmax over both: brute force on the pieces."""
    c, inv, q, kt, vt = _tail_case(2, 7)
    Pi = rotation(5, 16)
    K = att.decode_cell(c["cells"][0][0], 0, 16, Pi)
    V = att.decode_cell(c["cells"][0][1], 0, 16, Pi)
    qr = rope(q, 40, inv)
    want = att.decode_layer_tail(c, 0, q, 40, inv, 0.3, kt, vt)
    for j in range(4):
        h = j // 2
        parts = []
        for Kx, Vx in ((rope(K[h], np.arange(40), inv), V[h]), (kt[h], vt[h])):
            s = 0.3 * Kx @ qr[j]
            m = s.max()
            p = np.exp(s - m)
            parts.append((m, p.sum(), p @ Vx))
        M = max(m for m, _, _ in parts)
        num = sum(np.exp(m - M) * o for m, _, o in parts)
        den = sum(np.exp(m - M) * l for m, l, _ in parts)
        assert np.allclose(num / den, want[j], rtol=1e-12, atol=1e-12)
