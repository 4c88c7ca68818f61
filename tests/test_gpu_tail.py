"""GPU parity of decode attention over a compressed cache plus an
uncompressed tail (jolt_decode_attention_tail) against the oracle's single
softmax over both (oracle.attention.decode_layer_tail): the MFMA path and the
float32 path, bf16 and float32 tails, ragged tail lengths (0 included) in one
batch, and a tail longer than one split.  Tolerances as for the compressed
decode: rel-L2 <= 5e-3 and max-abs <= 2e-2 on the MFMA path, rel-L2 <= 1e-5
on the float32 path."""
import math

import numpy as np
import pytest

import compressed_cache_decode_jolt_amd as J
from oracle import attention as att
from oracle.compress import compress
from oracle.rope import rope
from workloads import gen, get_config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    J.lib()


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def tails(seed, B, H, cap, d, lens, Ts, inv, dtype):
    """Post-RoPE tail keys at positions T_b + i and values, rounded to the
    tail dtype; rows past tail_len are filled with garbage (never read)."""
    g = np.random.default_rng(seed)
    K = np.full((B, H, cap, d), 1e4)
    V = np.full((B, H, cap, d), -1e4)
    for b in range(B):
        n = lens[b]
        pos = Ts[b] + np.arange(n)
        K[b, :, :n] = rope(g.standard_normal((H, n, d)) * 1.3, pos, inv)
        V[b, :, :n] = g.standard_normal((H, n, d)) * 3.0
    if dtype == "bf16":
        K, V = gen.to_bf16_values(K).astype(np.float64), gen.to_bf16_values(V).astype(np.float64)
    return K, V


def run(caches, layer, q, q_pos, inv, scale, K, V, lens, dtype, kernel=None, split=0,
        q_dtype=torch.bfloat16):
    hs = [J.jolt_load_cache(c) for c in caches]
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qt = torch.from_numpy(q.astype(np.float32)).to(q_dtype).cuda()
    kt = torch.from_numpy(K.astype(np.float32)).to(dt).cuda()
    vt = torch.from_numpy(V.astype(np.float32)).to(dt).cuda()
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    nb = J.jolt_decode_tail_workspace_size(hs, layer, K.shape[2], kernel=kernel, split_tokens=split)
    ws = torch.full((nb,), 0x7F, dtype=torch.uint8, device="cuda")
    J.jolt_decode_attention_tail(hs, layer, qt, q_pos, inv, scale, kt, vt, lens, out, ws,
                                 kernel=kernel, split_tokens=split)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kernel", [J.KERNEL_MFMA, J.KERNEL_GENERIC])
def test_tail_batch_ragged(kernel, dtype):
    d, H, H_q = 128, 2, 8
    spec = [(300, (48, 32, 4), (64, 32, 2), 17), (700, (64, 64, 8), (96, 64, 8), 0),
            (513, (32, 16, 2), (32, 32, 4), 200), (1000, (96, 64, 0), (64, 32, 8), 64)]
    caches = [gen.small_cache(180 + i, T, H, H_q, d, [(aK, aV)], [1])
              for i, (T, aK, aV, _) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(5e5, d)
    lens = [n for *_, n in spec]
    Ts = [T for T, *_ in spec]
    K, V = tails(181, len(spec), H, 200, d, lens, Ts, inv, dtype)
    q = np.stack([gen.queries(182, i, 0, H_q, d, "bf16") for i in range(len(spec))])
    q_pos = [T + n for T, n in zip(Ts, lens)]
    got = run(caches, 0, q, q_pos, inv, 0.088, K, V, lens, dtype, kernel=kernel)
    rt, at = (5e-3, 2e-2) if kernel == J.KERNEL_MFMA else (1e-5, 1e-4)
    for b in range(len(spec)):
        want = att.decode_layer_tail(caches[b], 0, q[b].astype(np.float64), q_pos[b], inv, 0.088,
                                     K[b, :, :lens[b]], V[b, :, :lens[b]])
        r, mx = rel_l2(got[b], want), float(np.max(np.abs(got[b] - want)))
        assert r <= rt and mx <= at, (b, r, mx)


def test_tail_on_llama8b_layer_one_query_and_long_tail():
    """The 4K-token layer (oracle-compressed at its 3x allocation) with a
    2000-token bf16 tail (several tail splits), then the MHA head shape
    (one query per KV head) with a short tail."""
    import json, os
    cfg = get_config(1)
    alloc = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "allocations.json")))
    (aK, aV), = alloc["1"]["tables"]["3x"]["groups"]
    X = (gen.kv_group(cfg, 0, 0, 0), gen.kv_group(cfg, 0, 0, 1))
    c = compress([X], [(tuple(aK), tuple(aV))], "bf16", 0x4A4F4C54, cfg.H_q, cfg.group_start())
    inv = gen.rope_inv_freq_input(cfg.rope_base, cfg.d)
    K, V = tails(183, 1, cfg.H, 2000, cfg.d, [2000], [cfg.T], inv, "bf16")
    q = gen.cfg_queries(cfg, 0, 0)[None]
    qp = [cfg.T + 2000]
    got = run([c], 0, q, qp, inv, 1 / math.sqrt(cfg.d), K, V, [2000], "bf16")
    want = att.decode_layer_tail(c, 0, q[0].astype(np.float64), qp[0], inv, 1 / math.sqrt(cfg.d),
                                 K[0], V[0])
    assert rel_l2(got[0], want) <= 5e-3 and np.max(np.abs(got[0] - want)) <= 2e-2
    # one query per KV head
    d, H = 128, 4
    c = gen.small_cache(184, 900, H, H, d, [((320, 64, 2), (160, 64, 8))], [1])
    inv = gen.rope_inv_freq_input(1e4, d)
    K, V = tails(185, 1, H, 40, d, [33], [900], inv, "bf16")
    q = gen.queries(186, 0, 0, H, d, "bf16")[None]
    got = run([c], 0, q, [933], inv, 0.088, K, V, [33], "bf16")
    want = att.decode_layer_tail(c, 0, q[0].astype(np.float64), 933, inv, 0.088, K[0, :, :33],
                                 V[0, :, :33])
    assert rel_l2(got[0], want) <= 5e-3 and np.max(np.abs(got[0] - want)) <= 2e-2


def test_tail_on_fp32_workload():
    cfg = get_config(0)
    X = (gen.kv_group(cfg, 0, 0, 0), gen.kv_group(cfg, 0, 0, 1))
    c = compress([X], [(cfg.fixed, cfg.fixed)], "f32", 0x4A4F4C54, cfg.H_q, cfg.group_start())
    inv = gen.rope_inv_freq_input(cfg.rope_base, cfg.d)
    K, V = tails(187, 1, cfg.H, 70, cfg.d, [70], [cfg.T], inv, "f32")
    q = gen.cfg_queries(cfg, 0, 0)[None]
    got = run([c], 0, q, [cfg.T + 70], inv, 0.125, K, V, [70], "f32", q_dtype=torch.float32)
    want = att.decode_layer_tail(c, 0, q[0].astype(np.float64), cfg.T + 70, inv, 0.125, K[0], V[0])
    assert rel_l2(got[0], want) <= 1e-5
