"""GPU parity of the second value pass (one query per KV head, key ranks up
to 256, value ranks above 128): the split kernel writes every token's logit
and the residual part of the output, the merge the final softmax statistics,
then value_gemm / value_finish add W2_V (sum_t p_t A_V[t]) for all heads.
Against the oracle's decode of the same caches, at the MFMA tolerances
(rel-L2 <= 5e-3, max-abs <= 2e-2):

* one launch class whose sequences have different value ranks, one of them
  0 (no value factor: the second pass skips it) and ragged lengths, with
  short splits, with splits of 1024 tokens (two 16-token blocks per wave
  step in the split kernel) and with one split per sequence (the split
  kernel then writes the output and the statistics itself, no merge);
* more than 32 sequences (two batch chunks: the logits, statistics and
  partial sums at the second chunk's offsets);
* an uncompressed tail under the same softmax;
* the fixed block schedule (bitwise repeatable through both passes);
* the allocation-free entry point, which keeps the single pass, against the
  workspace entry point on the same call;
* 20 KV heads (a partly empty second 16-head group) and 40 (above the pass's
  32: the single pass);
* key ranks above 256: 8 waves with Pi in LDS where W2_K and Pi fit there
  (ranks 320 without a key residual, 384 and 448 with one; any value rank,
  and a sequence without a value factor in the same launch), the 4-wave
  single pass where they do not (rank 512 with 8-bit keys).
"""
import numpy as np
import pytest

import compressed_cache_decode_jolt_amd as J
from oracle import attention as att
from oracle.rope import rope
from workloads import gen

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    J.lib()


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def decode(caches, q, q_pos, inv, scale, deterministic=False, noalloc=False, split=0):
    hs = [J.jolt_load_cache(c) for c in caches]
    qt = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).cuda()
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        J.jolt_decode_attention_noalloc(hs, 0, qt, q_pos, inv, scale, out, kernel=J.KERNEL_MFMA,
                                        deterministic=deterministic)
    else:
        nb = J.jolt_decode_workspace_size(hs, 0, kernel=J.KERNEL_MFMA, split_tokens=split)
        ws = torch.full((nb,), 0x7F, dtype=torch.uint8, device="cuda")  # no zeroed buffers
        J.jolt_decode_attention(hs, 0, qt, q_pos, inv, scale, out, ws, kernel=J.KERNEL_MFMA,
                                split_tokens=split, deterministic=deterministic)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check(got, caches, q, q_pos, inv, scale):
    want = att.decode_attention(caches, 0, np.asarray(q, np.float64), q_pos, inv, scale)
    for b in range(len(caches)):
        r, mx = rel_l2(got[b], want[b]), float(np.max(np.abs(got[b] - want[b])))
        assert r <= 5e-3 and mx <= 2e-2, (b, r, mx)


@pytest.mark.parametrize("split", [0, 1024, 2048])
def test_class_with_mixed_value_ranks(split):
    d, H = 128, 4
    # same key bits, key rank and value bits: one launch class; value ranks
    # 400, 0, 160, 288
    spec = [(700, (160, 64, 8), (400, 96, 4)), (333, (160, 48, 8), (0, 0, 4)),
            (1100, (160, 64, 8), (160, 64, 4)), (450, (160, 32, 8), (288, 80, 4))]
    caches = [gen.small_cache(300 + i, T, H, H, d, [(aK, aV)], [1])
              for i, (T, aK, aV) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(1e4, d)
    q = np.stack([gen.queries(301, i, 0, H, d, "bf16") for i in range(len(spec))])
    q_pos = [T for T, _, _ in spec]
    check(decode(caches, q, q_pos, inv, 0.088, split=split), caches, q, q_pos, inv, 0.088)


def test_two_batch_chunks():
    d, H = 128, 2
    ranks = [(96, 64, 4), (64, 32, 2)]
    spec = [(200 + 37 * i, ranks[i % 2], (160 + 16 * (i % 5), 48, (0, 2, 4, 8)[i % 4]))
            for i in range(40)]
    caches = [gen.small_cache(400 + i, T, H, H, d, [(aK, aV)], [1])
              for i, (T, aK, aV) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(1e4, d)
    q = np.stack([gen.queries(401, i, 0, H, d, "bf16") for i in range(len(spec))])
    q_pos = [T for T, _, _ in spec]
    check(decode(caches, q, q_pos, inv, 0.088), caches, q, q_pos, inv, 0.088)


def test_with_an_uncompressed_tail():
    d, H, cap = 128, 4, 96
    spec = [(900, (192, 64, 4), (448, 96, 8), 96), (400, (192, 48, 4), (256, 64, 2), 0),
            (1300, (192, 64, 4), (320, 64, 4), 33)]
    caches = [gen.small_cache(500 + i, T, H, H, d, [(aK, aV)], [1])
              for i, (T, aK, aV, _) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(1e4, d)
    g = np.random.default_rng(501)
    lens = [n for *_, n in spec]
    K = np.zeros((len(spec), H, cap, d))
    V = np.zeros((len(spec), H, cap, d))
    for b, (T, _, _, n) in enumerate(spec):
        K[b, :, :n] = rope(g.standard_normal((H, n, d)) * 1.3, T + np.arange(n), inv)
        V[b, :, :n] = g.standard_normal((H, n, d)) * 3.0
    K, V = gen.to_bf16_values(K).astype(np.float64), gen.to_bf16_values(V).astype(np.float64)
    q = np.stack([gen.queries(502, i, 0, H, d, "bf16") for i in range(len(spec))])
    q_pos = [T + n for T, _, _, n in spec]
    hs = [J.jolt_load_cache(c) for c in caches]
    qt = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).cuda()
    kt = torch.from_numpy(K.astype(np.float32)).to(torch.bfloat16).cuda()
    vt = torch.from_numpy(V.astype(np.float32)).to(torch.bfloat16).cuda()
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    nb = J.jolt_decode_tail_workspace_size(hs, 0, cap, kernel=J.KERNEL_MFMA)
    ws = torch.full((nb,), 0x7F, dtype=torch.uint8, device="cuda")
    J.jolt_decode_attention_tail(hs, 0, qt, q_pos, inv, 0.088, kt, vt, lens, out, ws,
                                 kernel=J.KERNEL_MFMA)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    for b in range(len(spec)):
        want = att.decode_layer_tail(caches[b], 0, q[b].astype(np.float64), q_pos[b], inv, 0.088,
                                     K[b, :, :lens[b]], V[b, :, :lens[b]])
        r, mx = rel_l2(got[b], want), float(np.max(np.abs(got[b] - want)))
        assert r <= 5e-3 and mx <= 2e-2, (b, r, mx)


def test_fixed_schedule_is_bitwise_repeatable_and_noalloc_agrees():
    d, H = 128, 4
    spec = [(1500, (128, 64, 2), (384, 96, 4)), (777, (128, 64, 2), (208, 64, 8))]
    caches = [gen.small_cache(600 + i, T, H, H, d, [(aK, aV)], [1])
              for i, (T, aK, aV) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(1e4, d)
    q = np.stack([gen.queries(601, i, 0, H, d, "bf16") for i in range(len(spec))])
    q_pos = [T for T, _, _ in spec]
    a = decode(caches, q, q_pos, inv, 0.088, deterministic=True)
    b = decode(caches, q, q_pos, inv, 0.088, deterministic=True)
    assert np.array_equal(a, b)
    check(a, caches, q, q_pos, inv, 0.088)
    # the allocation-free entry point keeps the value factors in the split
    # kernel: a different summation, the same result within the tolerance
    c = decode(caches, q, q_pos, inv, 0.088, noalloc=True)
    check(c, caches, q, q_pos, inv, 0.088)
    assert rel_l2(c, a) <= 5e-3


@pytest.mark.parametrize("H", [20, 40])
def test_head_counts_around_the_two_head_groups(H):
    """20 KV heads: the second 16-head group of the value product is partly
    empty; 40 heads: more than the pass's 32, so the call keeps the single
    pass.  Either way the oracle's result."""
    d = 128
    spec = [(600, (96, 64, 4), (224, 64, 2)), (1000, (96, 48, 4), (160, 48, 2))]
    caches = [gen.small_cache(700 + 10 * H + i, T, H, H, d, [(aK, aV)], [1])
              for i, (T, aK, aV) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(1e4, d)
    q = np.stack([gen.queries(701, i, 0, H, d, "bf16") for i in range(len(spec))])
    q_pos = [T for T, _, _ in spec]
    check(decode(caches, q, q_pos, inv, 0.088), caches, q, q_pos, inv, 0.088)


@pytest.mark.parametrize("aK, aV", [((320, 96, 0), (256, 32, 4)), ((384, 32, 2), (192, 96, 8)),
                                    ((448, 64, 4), (160, 64, 2)), ((448, 64, 4), (64, 32, 2)),
                                    ((384, 32, 8), (32, 16, 4)), ((512, 96, 8), (224, 48, 4))])
def test_wide_key_ranks(aK, aV):
    d, H = 128, 4
    rv2 = aV[0] - 32  # the second sequence's value rank (0: no value factor)
    spec = [(1400, aK, aV), (700, (aK[0], aK[1] // 2, aK[2]), (rv2, aV[1] if rv2 else 0, aV[2]))]
    caches = [gen.small_cache(800 + aK[0] + i, T, H, H, d, [(k, v)], [1])
              for i, (T, k, v) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(1e4, d)
    q = np.stack([gen.queries(801, i, 0, H, d, "bf16") for i in range(len(spec))])
    q_pos = [T for T, _, _ in spec]
    check(decode(caches, q, q_pos, inv, 0.088), caches, q, q_pos, inv, 0.088)
    check(decode(caches, q, q_pos, inv, 0.088, split=512), caches, q, q_pos, inv, 0.088)
