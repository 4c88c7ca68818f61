"""GPU parity: the HIP decode path (through the C ABI) against the oracle.

Every case feeds the same seeded compressed cache to both sides and compares
element by element:
  * float32 caches (the tiny workload): rel-L2 <= 1e-5;
  * bf16 caches, generic kernel (fp32 arithmetic): rel-L2 <= 1e-5;
  * bf16 caches, MFMA kernel: rel-L2 <= 5e-3 and max-abs <= 2e-2;
  * residual codes read back from the device layout: bit-exact.
"""
import math

import numpy as np
import pytest

import compressed_cache_decode_jolt_amd as J
from oracle import attention as att
from oracle.compress import compress
from oracle.quant import unpack
from oracle.rope import rope
from oracle.rotation import rotation
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


def run_decode(caches, layer, q, q_pos, inv, scale, q_dtype="bf16", kernel=None, split=0,
               handles=None, ws=None):
    hs = handles or [J.jolt_load_cache(c) for c in caches]
    dt = torch.bfloat16 if q_dtype == "bf16" else torch.float32
    qt = torch.from_numpy(np.asarray(q, dtype=np.float32)).to(dt).cuda()
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    nb = J.jolt_decode_workspace_size(hs, layer, kernel=kernel, split_tokens=split)
    if ws is None:
        ws = torch.zeros(max(nb, 1), dtype=torch.uint8, device="cuda")
    assert ws.numel() >= nb
    J.jolt_decode_attention(hs, layer, qt, q_pos, inv, scale, out, ws, kernel=kernel,
                            split_tokens=split)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def oracle_decode(caches, layer, q, q_pos, inv, scale):
    return att.decode_attention(caches, layer, np.asarray(q, np.float64), q_pos, inv, scale)


KERNELS = [J.KERNEL_GENERIC, J.KERNEL_MFMA]


def tol(kernel, f32):
    if kernel == J.KERNEL_MFMA:
        return 5e-3, 2e-2
    return 1e-5, 1e-4


# ------------------------------------------------------------ bit-exact --
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("T", [1, 37, 300])
def test_unpack_bit_exact(bits, T):
    r = min(T, 16)
    c = gen.small_cache(bits, T, 3, 6, 128, [((r, 16, bits), (min(T, 32), 16, bits))], [2])
    h = J.jolt_load_cache(c)
    for layer in range(2):
        for tau in range(2):
            got = J.jolt_debug_unpack(h, layer, tau)
            want = unpack(c["cells"][0][tau]["codes"][layer], bits, 128)
            assert np.array_equal(got, want)


def test_unpack_d64_oracle_codes():
    cfg = get_config(0)
    groups = [(gen.kv_group(cfg, 0, 0, 0), gen.kv_group(cfg, 0, 0, 1))]
    c = compress(groups, [((32, 16, 4), (32, 16, 2))], "f32", 7, cfg.H_q, [0, 1])
    h = J.jolt_load_cache(c)
    for tau, b in ((0, 4), (1, 2)):
        assert np.array_equal(J.jolt_debug_unpack(h, 0, tau),
                              unpack(c["cells"][0][tau]["codes"][0], b, 64))


# ------------------------------------------------------------- workloads --
def tiny_cache():
    cfg = get_config(0)
    groups = [(gen.kv_group(cfg, 0, 0, 0), gen.kv_group(cfg, 0, 0, 1))]
    return cfg, compress(groups, [(cfg.fixed, cfg.fixed)], "f32", 0x4A4F4C54, cfg.H_q,
                         cfg.group_start())


def test_tiny_fp32_workload():
    cfg, c = tiny_cache()
    inv = gen.rope_inv_freq_input(cfg.rope_base, cfg.d)
    q = gen.cfg_queries(cfg, 0, 0)[None]
    scale = 1 / math.sqrt(cfg.d)
    got = run_decode([c], 0, q, [cfg.T], inv, scale, "f32")
    want = oracle_decode([c], 0, q, [cfg.T], inv, scale)
    assert rel_l2(got, want) <= 1e-5, rel_l2(got, want)


def layer8b_cache():
    cfg = get_config(1)
    import json, os
    alloc = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "allocations.json")))
    (aK, aV), = alloc["1"]["tables"]["3x"]["groups"]
    groups = [(gen.kv_group(cfg, 0, 0, 0), gen.kv_group(cfg, 0, 0, 1))]
    return cfg, compress(groups, [(tuple(aK), tuple(aV))], "bf16", 0x4A4F4C54, cfg.H_q,
                         cfg.group_start())


@pytest.fixture(scope="module")
def l8b():
    return layer8b_cache()


@pytest.mark.parametrize("kernel", [None] + KERNELS)
def test_llama8b_layer_workload(l8b, kernel):
    cfg, c = l8b
    inv = gen.rope_inv_freq_input(cfg.rope_base, cfg.d)
    q = gen.cfg_queries(cfg, 0, 0)[None]
    scale = 1 / math.sqrt(cfg.d)
    got = run_decode([c], 0, q, [cfg.T], inv, scale, kernel=kernel)
    want = oracle_decode([c], 0, q, [cfg.T], inv, scale)
    r, mx = rel_l2(got, want), float(np.max(np.abs(got - want)))
    print(f"llama8b layer kernel={kernel}: rel_l2={r:.3e} max_abs={mx:.3e}")
    # the automatic choice here is the MFMA kernel
    rt, at = tol(J.KERNEL_MFMA if kernel is None else kernel, False)
    assert r <= rt and mx <= at


# ------------------------------------------------------------- coverage --
BITS = [0, 2, 4, 8]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("bK", BITS)
@pytest.mark.parametrize("bV", BITS)
def test_bits_matrix_ragged(bK, bV, kernel):
    T, H, H_q, d = 300, 2, 8, 128
    c = gen.small_cache(10 * bK + bV, T, H, H_q, d, [((40, 24, bK), (33, 17, bV))], [1])
    inv = gen.rope_inv_freq_input(5e5, d)
    q = gen.queries(77, bK, bV, H_q, d, "bf16")[None]
    got = run_decode([c], 0, q, [T], inv, 0.09, kernel=kernel)
    want = oracle_decode([c], 0, q, [T], inv, 0.09)
    r, a = tol(kernel, False)
    assert rel_l2(got, want) <= r and np.max(np.abs(got - want)) <= a


@pytest.mark.parametrize("kernel", KERNELS)
def test_split_invariance(kernel):
    """The same call at several split sizes; 1024 tokens is one split for the
    whole sequence (on the MFMA path the split kernel then writes the output
    itself and no merge runs), also checked against the oracle."""
    T = 1000
    c = gen.small_cache(5, T, 4, 16, 128, [((64, 32, 4), (96, 64, 2))], [1])
    inv = gen.rope_inv_freq_input(1e4, 128)
    q = gen.queries(78, 0, 0, 16, 128, "bf16")[None]
    hs = [J.jolt_load_cache(c)]
    outs = [run_decode([c], 0, q, [T], inv, 0.1, kernel=kernel, split=s, handles=hs)
            for s in (0, 128, 256, 1024)]
    for o in outs[1:]:
        assert rel_l2(o, outs[0]) <= (2e-6 if kernel == J.KERNEL_GENERIC else 2e-3)
    want = oracle_decode([c], 0, q, [T], inv, 0.1)
    r, a = tol(kernel, False)
    assert rel_l2(outs[-1][0], want[0]) <= r and np.max(np.abs(outs[-1][0] - want[0])) <= a


@pytest.mark.parametrize("kernel", KERNELS)
def test_batch_of_different_lengths_and_ranks_same_bits(kernel):
    d, H, H_q = 128, 2, 4
    caches = [gen.small_cache(50 + i, T, H, H_q, d, [(aK, aV)], [1])
              for i, (T, aK, aV) in enumerate([(100, (16, 16, 4), (16, 16, 2)),
                                                (257, (48, 32, 4), (64, 32, 2)),
                                                (1000, (96, 64, 4), (128, 96, 2))])]
    inv = gen.rope_inv_freq_input(5e5, d)
    q = np.stack([gen.queries(83, i, 0, H_q, d, "bf16") for i in range(3)])
    q_pos = [100, 300, 1000]
    got = run_decode(caches, 0, q, q_pos, inv, 0.088, kernel=kernel)
    want = oracle_decode(caches, 0, q, q_pos, inv, 0.088)
    r, a = tol(kernel, False)
    for b in range(3):
        assert rel_l2(got[b], want[b]) <= r
        assert np.max(np.abs(got[b] - want[b])) <= a and np.max(np.abs(got[b] - want[b])) <= a


@pytest.mark.parametrize("split", [0, 128])
def test_mixed_bits_batch_on_mfma(split):
    """Sequences whose layer has different key/value bit-widths (per-sequence
    allocations) share one call: one MFMA launch per bit class, one merge."""
    d, H, H_q = 128, 2, 8
    spec = [(300, (16, 16, 2), (16, 16, 4)), (513, (32, 16, 8), (48, 32, 4)),
            (77, (16, 16, 2), (16, 16, 4)), (1000, (64, 64, 0), (32, 64, 8)),
            (256, (48, 32, 4), (160, 64, 2))]
    caches = [gen.small_cache(60 + i, T, H, H_q, d, [(aK, aV)], [1])
              for i, (T, aK, aV) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(5e5, d)
    q = np.stack([gen.queries(61, i, 0, H_q, d, "bf16") for i in range(len(spec))])
    q_pos = [T for T, _, _ in spec]
    got = run_decode(caches, 0, q, q_pos, inv, 0.088, kernel=J.KERNEL_MFMA, split=split)
    want = oracle_decode(caches, 0, q, q_pos, inv, 0.088)
    for b in range(len(spec)):
        assert rel_l2(got[b], want[b]) <= 5e-3, (b, rel_l2(got[b], want[b]))
        assert np.max(np.abs(got[b] - want[b])) <= 2e-2


WIDE_KEYS = [((320, 64, 0), (64, 32, 2)), ((384, 32, 2), (128, 48, 8)),
             ((448, 64, 4), (128, 64, 0)), ((512, 96, 8), (64, 32, 4))]


@pytest.mark.parametrize("split", [0, 128])
@pytest.mark.parametrize("aK,aV", WIDE_KEYS, ids=[f"K{k[0]}b{k[2]}-V{v[0]}b{v[2]}" for k, v in WIDE_KEYS])
def test_wide_key_ranks_on_mfma(aK, aV, split):
    """Key ranks above 256 (the MHA workload's wide groups): W2_K alone in
    LDS, Pi's fragments in registers, 4 waves; every residual width."""
    d, H, H_q, T = 128, 4, 16, 700
    c = gen.small_cache(90 + aK[0] // 64, T, H, H_q, d, [(aK, aV)], [1])
    inv = gen.rope_inv_freq_input(5e5, d)
    q = gen.queries(91, aK[2], aV[2], H_q, d, "bf16")[None]
    got = run_decode([c], 0, q, [T], inv, 0.088, kernel=J.KERNEL_MFMA, split=split)
    want = oracle_decode([c], 0, q, [T], inv, 0.088)
    r, mx = rel_l2(got, want), float(np.max(np.abs(got - want)))
    assert r <= 5e-3 and mx <= 2e-2, (r, mx)


def test_grouped_wide_keys_with_wide_values_take_the_float32_kernel():
    """Grouped queries with key ranks above 256 and value ranks above 128 are
    not an MFMA class (it would not fit a SIMD's registers): forcing the MFMA
    kernel is refused, the automatic choice runs the float32 kernel and
    matches the oracle at its tolerance."""
    d, H, H_q, T = 128, 4, 16, 700
    c = gen.small_cache(97, T, H, H_q, d, [((384, 32, 2), (192, 48, 8))], [1])
    inv = gen.rope_inv_freq_input(5e5, d)
    q = gen.queries(91, 2, 8, H_q, d, "bf16")[None]
    h = J.jolt_load_cache(c)
    with pytest.raises(J.JoltError):
        J.jolt_decode_workspace_size([h], 0, kernel=J.KERNEL_MFMA)
    got = run_decode([c], 0, q, [T], inv, 0.088, handles=[h])
    want = oracle_decode([c], 0, q, [T], inv, 0.088)
    assert rel_l2(got, want) <= 1e-5


ONE_QUERY = [((64, 64, 0), (320, 64, 4)), ((192, 48, 8), (512, 96, 2)),
             ((256, 64, 2), (144, 32, 8)), ((320, 64, 4), (256, 96, 4)),
             ((448, 32, 0), (96, 32, 8)), ((512, 96, 8), (48, 32, 0)),
             ((384, 64, 2), (0, 0, 8)), ((128, 64, 0), (0, 0, 4))]


@pytest.mark.parametrize("split", [0, 128])
@pytest.mark.parametrize("aK,aV", ONE_QUERY, ids=[f"K{k[0]}b{k[2]}-V{v[0]}b{v[2]}" for k, v in ONE_QUERY])
def test_one_query_per_kv_head_on_mfma(aK, aV, split):
    """One query per KV head (the MHA workload's shape) in the 4-wave
    classes: value ranks above 128, and key ranks above 256 with value ranks
    up to 256; the value products run as dot products on the VALU."""
    d, H, H_q, T = 128, 4, 4, 700
    c = gen.small_cache(120 + aK[0] // 32 + aV[0] // 16, T, H, H_q, d, [(aK, aV)], [1])
    inv = gen.rope_inv_freq_input(1e4, d)
    q = gen.queries(121, aK[2], aV[2], H_q, d, "bf16")[None]
    got = run_decode([c], 0, q, [T], inv, 0.088, kernel=J.KERNEL_MFMA, split=split)
    want = oracle_decode([c], 0, q, [T], inv, 0.088)
    r, mx = rel_l2(got, want), float(np.max(np.abs(got - want)))
    assert r <= 5e-3 and mx <= 2e-2, (r, mx)


@pytest.mark.parametrize("H,H_q,aK,aV", [(2, 8, (96, 64, 4), (64, 32, 4)),
                                         (4, 4, (320, 64, 8), (160, 64, 2))],
                         ids=["group4", "one-query-wide"])
def test_fp32_queries_on_mfma(H, H_q, aK, aV):
    """float32 queries (converted in the kernel's prologue) at a decode
    position past the cache's end, on an 8-wave class and a one-query
    4-wave class."""
    d, T = 128, 600
    c = gen.small_cache(140 + H, T, H, H_q, d, [(aK, aV)], [1])
    inv = gen.rope_inv_freq_input(5e5, d)
    q = gen.queries(141, H, 0, H_q, d, "f32")[None]
    got = run_decode([c], 0, q, [T + 37], inv, 0.088, q_dtype="f32", kernel=J.KERNEL_MFMA)
    want = oracle_decode([c], 0, q, [T + 37], inv, 0.088)
    r, mx = rel_l2(got, want), float(np.max(np.abs(got - want)))
    assert r <= 5e-3 and mx <= 2e-2, (r, mx)


@pytest.mark.parametrize("split", [512, 1024])
def test_two_blocks_per_step_on_short_key_chains(split):
    """Key ranks up to 64 with long splits take two 16-token blocks per wave
    step; a batch of such classes (ragged lengths, a split's last step half
    empty) against the oracle."""
    d, H, H_q = 128, 2, 8
    spec = [(1500, (48, 32, 4), (64, 32, 2)), (1111, (20, 16, 8), (40, 32, 4)),
            (900, (0, 0, 4), (64, 48, 8)), (1500, (64, 64, 2), (16, 16, 0))]
    caches = [gen.small_cache(150 + i, T, H, H_q, d, [(aK, aV)], [1])
              for i, (T, aK, aV) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(5e5, d)
    q = np.stack([gen.queries(151, i, 0, H_q, d, "bf16") for i in range(len(spec))])
    q_pos = [T for T, _, _ in spec]
    got = run_decode(caches, 0, q, q_pos, inv, 0.088, kernel=J.KERNEL_MFMA, split=split)
    want = oracle_decode(caches, 0, q, q_pos, inv, 0.088)
    for b in range(len(spec)):
        assert rel_l2(got[b], want[b]) <= 5e-3, (b, rel_l2(got[b], want[b]))
        assert np.max(np.abs(got[b] - want[b])) <= 2e-2


@pytest.mark.parametrize("split", [0, 256])
def test_one_query_batch_of_mixed_classes(split):
    """One query per KV head, one batch whose sequences fall in different
    launch classes and lengths: 8 waves (value ranks up to 64), the one-query
    8-wave class for value ranks above 128, and the one-query 4-wave class
    for key ranks above 256."""
    d, H, H_q = 128, 4, 4
    spec = [(300, (96, 64, 4), (64, 32, 2)), (1000, (160, 64, 8), (400, 96, 4)),
            (400, (352, 96, 2), (128, 64, 8)), (513, (96, 64, 4), (64, 32, 2))]
    caches = [gen.small_cache(130 + i, T, H, H_q, d, [(aK, aV)], [1])
              for i, (T, aK, aV) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(1e4, d)
    q = np.stack([gen.queries(131, i, 0, H_q, d, "bf16") for i in range(len(spec))])
    q_pos = [T for T, _, _ in spec]
    got = run_decode(caches, 0, q, q_pos, inv, 0.088, kernel=J.KERNEL_MFMA, split=split)
    want = oracle_decode(caches, 0, q, q_pos, inv, 0.088)
    for b in range(len(spec)):
        assert rel_l2(got[b], want[b]) <= 5e-3, (b, rel_l2(got[b], want[b]))
        assert np.max(np.abs(got[b] - want[b])) <= 2e-2


@pytest.mark.parametrize("kernel", KERNELS)
def test_batch_of_different_lengths_and_ranks(kernel):
    d, H, H_q = 128, 2, 4
    caches = [gen.small_cache(20 + i, T, H, H_q, d, [(aK, aV)], [1])
              for i, (T, aK, aV) in enumerate([(100, (16, 16, 2), (16, 16, 8)),
                                                (257, (48, 32, 4), (64, 32, 4)),
                                                (1000, (32, 64, 0), (128, 96, 2))])]
    inv = gen.rope_inv_freq_input(5e5, d)
    q = np.stack([gen.queries(79, i, 0, H_q, d, "bf16") for i in range(3)])
    q_pos = [100, 300, 1000]
    got = run_decode(caches, 0, q, q_pos, inv, 0.088, kernel=kernel)
    want = oracle_decode(caches, 0, q, q_pos, inv, 0.088)
    r, a = tol(kernel, False)
    for b in range(3):
        assert rel_l2(got[b], want[b]) <= r
        assert np.max(np.abs(got[b] - want[b])) <= a


@pytest.mark.parametrize("kernel", KERNELS)
def test_workspace_reused_across_calls(kernel):
    """One workspace, never cleared, serves consecutive calls with different
    shapes and split counts (stale partials of a longer call must not leak
    into a shorter one)."""
    d, H, H_q = 128, 4, 16
    ws = torch.full((1 << 22,), 0x7F, dtype=torch.uint8, device="cuda")
    inv = gen.rope_inv_freq_input(5e5, d)
    for i, (T, split) in enumerate([(700, 128), (2000, 256), (300, 0), (700, 128)]):
        c = gen.small_cache(70 + i, T, H, H_q, d, [((32, 32, 4), (64, 32, 2))], [1])
        q = gen.queries(84, i, 0, H_q, d, "bf16")[None]
        got = run_decode([c], 0, q, [T], inv, 0.1, kernel=kernel, split=split, ws=ws)
        want = oracle_decode([c], 0, q, [T], inv, 0.1)
        assert rel_l2(got, want) <= tol(kernel, False)[0], (i, rel_l2(got, want))
    # dense path on the same workspace
    g = np.random.default_rng(5)
    K = gen.to_bf16_values(g.standard_normal((1, H, 500, d))).astype(np.float64)
    V = gen.to_bf16_values(g.standard_normal((1, H, 500, d))).astype(np.float64)
    for _ in range(2):
        out = torch.empty((1, H_q, d), dtype=torch.float32, device="cuda")
        J.jolt_dense_attention(torch.from_numpy(K.astype(np.float32)).to(torch.bfloat16).cuda(),
                               torch.from_numpy(V.astype(np.float32)).to(torch.bfloat16).cuda(),
                               torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).cuda(),
                               [500], inv, 0.1, out, ws, split_tokens=64)
        torch.cuda.synchronize()
        want = att.dense_attention(K, V, q.astype(np.float64), [500], inv, 0.1)
        assert rel_l2(out.cpu().numpy(), want) <= 1e-5


@pytest.mark.parametrize("kernel", KERNELS)
def test_layer_groups(kernel):
    d, H, H_q, T = 128, 2, 8, 200
    c = gen.small_cache(30, T, H, H_q, d, [((32, 16, 4), (64, 32, 2)), ((16, 16, 8), (16, 32, 0))],
                        [3, 2])
    inv = gen.rope_inv_freq_input(5e5, d)
    hs = [J.jolt_load_cache(c)]
    for layer in range(5):
        q = gen.queries(80, 0, layer, H_q, d, "bf16")[None]
        got = run_decode([c], layer, q, [T], inv, 0.1, kernel=kernel, handles=hs)
        want = oracle_decode([c], layer, q, [T], inv, 0.1)
        assert rel_l2(got, want) <= tol(kernel, False)[0], layer


@pytest.mark.parametrize("kernel", KERNELS)
def test_degenerate_cases(kernel):
    d, H, H_q = 128, 1, 4
    r, _ = tol(kernel, False)
    inv = gen.rope_inv_freq_input(1e4, d)
    # T = 1: the output is V^_0 for every query head
    c = gen.small_cache(40, 1, H, H_q, d, [((1, 16, 4), (1, 16, 4))], [1])
    q = gen.queries(81, 0, 0, H_q, d, "bf16")[None]
    got = run_decode([c], 0, q, [0], inv, 0.1, kernel=kernel)
    assert rel_l2(got, oracle_decode([c], 0, q, [0], inv, 0.1)) <= r
    # no value factors and no value residual: the output is exactly 0
    c = gen.small_cache(41, 50, H, H_q, d, [((16, 16, 4), (0, 0, 0))], [1])
    got = run_decode([c], 0, q, [50], inv, 0.1, kernel=kernel)
    assert np.all(got == 0)
    # residual only (no Tucker part)
    c = gen.small_cache(42, 70, H, H_q, d, [((0, 0, 8), (0, 0, 2))], [1])
    got = run_decode([c], 0, q, [70], inv, 0.1, kernel=kernel)
    assert rel_l2(got, oracle_decode([c], 0, q, [70], inv, 0.1)) <= r
    # q = 0: uniform attention, the mean of V^
    c = gen.small_cache(43, 77, H, H_q, d, [((16, 16, 4), (32, 16, 4))], [1])
    got = run_decode([c], 0, np.zeros((1, H_q, d)), [77], inv, 0.1, kernel=kernel)
    Vh = att.decode_cell(c["cells"][0][1], 0, d, rotation(c["rotation_seed"], d))
    assert rel_l2(got[0], np.repeat(Vh.mean(axis=1), H_q // H, axis=0)) <= r


# ------------------------------------------------------------------ dense --
@pytest.mark.parametrize("d,H,H_q,T", [(128, 8, 32, 4096), (128, 2, 16, 333), (64, 2, 8, 256),
                                       (128, 4, 4, 1000)])
@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_dense_parity(d, H, H_q, T, kv):
    g = np.random.default_rng(T + d)
    inv = gen.rope_inv_freq_input(5e5, d)
    K = rope(g.standard_normal((2, H, T, d)) * 1.3, np.arange(T), inv)
    V = g.standard_normal((2, H, T, d)) * 3.0
    if kv == "bf16":
        K, V = gen.to_bf16_values(K).astype(np.float64), gen.to_bf16_values(V).astype(np.float64)
    q = np.stack([gen.queries(82, b, 0, H_q, d, "bf16") for b in range(2)]).astype(np.float64)
    dt = torch.bfloat16 if kv == "bf16" else torch.float32
    kt = torch.from_numpy(K.astype(np.float32)).to(dt).cuda()
    vt = torch.from_numpy(V.astype(np.float32)).to(dt).cuda()
    qt = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).cuda()
    out = torch.empty((2, H_q, d), dtype=torch.float32, device="cuda")
    ws = torch.zeros(J.jolt_dense_workspace_size(2, H, H_q, d, T), dtype=torch.uint8, device="cuda")
    J.jolt_dense_attention(kt, vt, qt, [T, T + 5], inv, 1 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    want = att.dense_attention(K, V, q, [T, T + 5], inv, 1 / math.sqrt(d))
    assert rel_l2(out.cpu().numpy(), want) <= 1e-5


# ------------------------------------------------------------------- trig --
@pytest.mark.parametrize("variant,bound", [(0, 1e-7), (1, 1e-6)])
def test_rope_sincos_accuracy(variant, bound):
    """The kernels' sine/cosine of every RoPE angle fl32(t * inv_freq_i),
    t = 0..65536, for both RoPE bases of the workloads, against float64.
    Variant 0 (polynomial) serves the float32 paths and query RoPE, variant 1
    (hardware units after a 2 pi reduction) the MFMA key path."""
    t = np.arange(65537, dtype=np.float32)
    worst = 0.0
    for base in (1e4, 5e5):
        inv = gen.rope_inv_freq_input(base, 128)
        ang = (t[:, None] * inv[None, :]).astype(np.float32).ravel()
        sn, cs = J.jolt_debug_sincos(ang, variant)
        a64 = ang.astype(np.float64)
        worst = max(worst, np.max(np.abs(sn - np.sin(a64))), np.max(np.abs(cs - np.cos(a64))))
    # the whole domain of the reduction: random float32 angles below 2^20
    big = (np.random.default_rng(0).random(200000) * 2 - 1).astype(np.float32) * np.float32(1048575.0)
    sn, cs = J.jolt_debug_sincos(big, variant)
    b64 = big.astype(np.float64)
    worst = max(worst, np.max(np.abs(sn - np.sin(b64))), np.max(np.abs(cs - np.cos(b64))))
    assert worst <= bound, worst


def test_rope_small_angle_blocks():
    """The key path's shortcut for frequency blocks whose angles stay at most
    128 rad over the launch: position * fl32(inv_freq / 2 pi) straight into the
    hardware units.  Against sin/cos of the float32 angle fl32(t * inv_freq)
    (float64) over every (position, frequency) with t * inv_freq <= 128, for
    both RoPE bases: within 2.5e-5 (three float32 roundings of a value below
    20.4 revolutions, plus the units' own error)."""
    worst = 0.0
    for base in (1e4, 5e5):
        inv = gen.rope_inv_freq_input(base, 128)
        t = np.arange(65537, dtype=np.float32)
        tt, ff = np.meshgrid(t, inv, indexing="ij")
        keep = tt.astype(np.float64) * ff.astype(np.float64) <= 128.0
        pairs = np.stack([tt[keep], ff[keep]], axis=1).astype(np.float32)
        sn, cs = J.jolt_debug_sincos(pairs, 2)
        a64 = (pairs[:, 0] * pairs[:, 1]).astype(np.float32).astype(np.float64)
        worst = max(worst, np.max(np.abs(sn - np.sin(a64))), np.max(np.abs(cs - np.cos(a64))))
    assert worst <= 2.5e-5, worst


@pytest.mark.parametrize("split", [512, 1024])
def test_one_query_two_blocks_per_step(split):
    """One query per KV head on the class with two 16-token blocks per wave
    step (key and value ranks up to 64, splits of at least 512 tokens),
    ragged lengths whose last split is short."""
    d, H, H_q = 128, 4, 4
    spec = [(1111, (48, 32, 4), (64, 32, 2)), (1500, (64, 64, 8), (32, 32, 8)),
            (700, (32, 16, 0), (16, 16, 4))]
    caches = [gen.small_cache(160 + i, T, H, H_q, d, [(aK, aV)], [1])
              for i, (T, aK, aV) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(1e4, d)
    q = np.stack([gen.queries(161, i, 0, H_q, d, "bf16") for i in range(len(spec))])
    q_pos = [T for T, _, _ in spec]
    got = run_decode(caches, 0, q, q_pos, inv, 0.088, kernel=J.KERNEL_MFMA, split=split)
    want = oracle_decode(caches, 0, q, q_pos, inv, 0.088)
    for b in range(len(spec)):
        assert rel_l2(got[b], want[b]) <= 5e-3, (b, rel_l2(got[b], want[b]))
        assert np.max(np.abs(got[b] - want[b])) <= 2e-2


@pytest.mark.parametrize("split", [256, 1024])
def test_one_query_wide_keys_long_splits(split):
    """One query per KV head with key ranks above 256 (4 waves, Pi's
    fragments in registers) over long splits: ragged lengths, residual-free
    and 2/4/8-bit keys, the three value classes."""
    d, H, H_q = 128, 4, 4
    spec = [(1111, (320, 64, 2), (160, 64, 8)), (1500, (384, 96, 8), (96, 32, 4)),
            (700, (448, 64, 0), (200, 64, 8)), (999, (512, 64, 0), (64, 32, 2)),
            (1300, (352, 64, 4), (256, 96, 4))]
    caches = [gen.small_cache(170 + i, T, H, H_q, d, [(aK, aV)], [1])
              for i, (T, aK, aV) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(1e4, d)
    q = np.stack([gen.queries(171, i, 0, H_q, d, "bf16") for i in range(len(spec))])
    q_pos = [T for T, _, _ in spec]
    got = run_decode(caches, 0, q, q_pos, inv, 0.088, kernel=J.KERNEL_MFMA, split=split)
    want = oracle_decode(caches, 0, q, q_pos, inv, 0.088)
    for b in range(len(spec)):
        assert rel_l2(got[b], want[b]) <= 5e-3, (b, rel_l2(got[b], want[b]))
        assert np.max(np.abs(got[b] - want[b])) <= 2e-2


DET_CASES = [(2, 8, 1500, (64, 32, 4), (48, 32, 2), 512),     # 8 waves, two blocks per step
             (2, 8, 2000, (96, 64, 8), (96, 64, 4), 0),       # 8 waves, value ranks <= 128
             (4, 4, 1300, (320, 64, 2), (160, 64, 8), 256),   # one query, wide keys, 4 waves
             (4, 4, 1300, (160, 64, 4), (400, 96, 4), 0),     # one query, value ranks > 128
             (2, 16, 900, (128, 64, 0), (256, 64, 2), 0)]     # 4 waves, value ranks > 128


@pytest.mark.parametrize("H,H_q,T,aK,aV,split", DET_CASES,
                         ids=["nb2", "v128", "hg1-widek", "hg1-widev", "wide-v"])
def test_deterministic_schedule_is_bitwise_repeatable(H, H_q, T, aK, aV, split):
    """With the fixed block schedule, repeated calls give identical output
    bytes (and stay within the tolerance of the oracle)."""
    d = 128
    c = gen.small_cache(170 + H + aK[0] // 16, T, H, H_q, d, [(aK, aV)], [1])
    inv = gen.rope_inv_freq_input(5e5, d)
    q = gen.queries(171, H, aK[0], H_q, d, "bf16")[None]
    h = J.jolt_load_cache(c)
    qt = torch.from_numpy(q).to(torch.bfloat16).cuda()
    nb = J.jolt_decode_workspace_size([h], 0, split_tokens=split)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(4):
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        J.jolt_decode_attention([h], 0, qt, [T], inv, 0.088, out, ws, split_tokens=split,
                                deterministic=True)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    want = oracle_decode([c], 0, q, [T], inv, 0.088)
    assert rel_l2(outs[0].astype(np.float64), want) <= 5e-3
