"""GPU parity of alignment-based layer grouping (jolt_flash_layer_groups)
against the oracle's (oracle.grouping), which follows the same steps in
float64 from the same seeded test matrix: identical group boundaries and
alignments within 1e-8, on generated caches whose layers share token bases
within known groups (the grouping must recover them), with a group-size cap,
and at the 64K stack's head shape."""
import numpy as np
import pytest

import compressed_cache_decode_jolt_amd as J
from oracle import grouping as gr
from workloads import gen, get_config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    J.lib()


def layers(n_groups, gs, H, T, d, seed, cfg=None):
    out = []
    for g in range(n_groups):
        if cfg is not None:
            XK, XV = (gen.kv_group(cfg, seed, g, tau, T=T) for tau in (0, 1))
        else:
            XK = gen.kv_tensor((89, seed, g, 0), gs, H, T, d, 1.0, True, 1, rank=16)
            XV = gen.kv_tensor((89, seed, g, 1), gs, H, T, d, 0.6, False, 0, rank=16)
        XK = gen.to_bf16_values(XK).astype(np.float64)
        XV = gen.to_bf16_values(XV).astype(np.float64)
        out += [(XK[l], XV[l]) for l in range(gs)]
    return out


def run(ls, r, tau, max_group=0):
    dev = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda()  # noqa: E731
    ks = [dev(k) for k, _ in ls]
    vs = [dev(v) for _, v in ls]
    return J.jolt_flash_layer_groups(ks, vs, r, tau, max_group, oversample=16, power_iters=2,
                                     sketch_seed=5)


@pytest.mark.parametrize("max_group", [0, 3])
def test_grouping_matches_oracle(max_group):
    ls = layers(3, 4, 2, 512, 64, 0)
    got_s, got_a = run(ls, 8, 0.5, max_group)
    want_s, want_a = gr.align_groups(ls, 8, 0.5, max_group, 16, 2, 5)
    assert got_s == want_s
    assert np.allclose(got_a, want_a, rtol=0, atol=1e-8)
    if max_group == 0:
        assert got_s == [0, 4, 8, 12]


def test_grouping_at_the_64k_head_shape():
    cfg = get_config(2)
    ls = layers(2, 4, cfg.H, 4096, cfg.d, 0, cfg=cfg)
    got_s, got_a = run(ls, 32, 0.5)
    want_s, want_a = gr.align_groups(ls, 32, 0.5, 0, 16, 2, 5)
    print("alignments:", np.round(got_a, 3))
    assert got_s == want_s == [0, 4, 8]
    assert np.allclose(got_a, want_a, rtol=0, atol=1e-8)
