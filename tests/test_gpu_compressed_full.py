"""GPU parity on caches produced by the oracle's compressor at full token
counts, with the residual widths the allocator picks for the long-context
workloads (8-bit keys and values, 2-bit values).

Unlike the synthetic stand-ins of test_gpu_full_size.py (random factors,
uniform codes, scales of a fixed fraction of the data), these cells carry
the residual scales a real compression produces: with 8-bit residuals the
quantiser steps are ~1e-3, which puts the softmax-weighted steps p * Delta
of the value path far below 1 and exercises the low end of the kernel's
fp16 operand range.  Each case compresses one layer group with
oracle.compress (exact ST-HOSVD, rotation, quantiser, packing), decodes it on
the GPU through the C ABI as bench.py does (automatic kernel and split) and
compares sampled (layer, KV head) rows with the oracle's decode:
rel-L2 <= 5e-3 and max-abs <= 2e-2 (bf16 factors, MFMA path).
"""
import math
import sys

import numpy as np
import pytest

import compressed_cache_decode_jolt_amd as J
from oracle import attention as att
from oracle.compress import compress
from oracle.rotation import rotation
from workloads import gen, get_config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    J.lib()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def compressed_group(cfg, group, alloc, T, seq=0):
    """One layer group of workload ``cfg`` (its spectra and outlier recipe for
    that group), T tokens, compressed by the oracle with (K, V) = alloc."""
    X = (gen.kv_group(cfg, seq, group, 0, T=T), gen.kv_group(cfg, seq, group, 1, T=T))
    cache = compress([X], [alloc], "bf16", 0x4A4F4C54, cfg.H_q, [0, cfg.group_size])
    del X
    return cache


# (workload, group whose spectra are used, (K, V) allocation, T, KV heads sampled, label)
CASES = [
    # the long-context stack at 2x: 8-bit keys and 8-bit values, full 64K tokens
    (2, 0, ((64, 80, 8), (64, 64, 8)), 65536, [0, 5], "llama3-8b-64k-2x"),
    # the 70B shape (8 query heads per KV head): 8-bit keys with 4-bit values, and
    # rank-192 4-bit keys
    (3, 0, ((64, 64, 8), (64, 128, 4)), 4096, [1, 6], "llama3-70b-k8"),
    (3, 1, ((192, 128, 4), (64, 128, 4)), 4096, [2, 7], "llama3-70b-k192"),
    # the MHA shape: 8-bit values with 2-bit keys, 8-bit keys with 2-bit values
    (4, 1, ((128, 48, 2), (448, 80, 8)), 4096, [0, 31], "mha-7b-v8"),
    (4, 3, ((256, 80, 8), (320, 48, 2)), 4096, [3, 17], "mha-7b-k8"),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg_idx,group,alloc,T,heads,label", CASES, ids=[c[-1] for c in CASES])
def test_compressed_group_decodes_like_oracle(cfg_idx, group, alloc, T, heads, label):
    cfg = get_config(cfg_idx)
    d, gs, Hg = cfg.d, cfg.group_size, cfg.H_q // cfg.H
    say(f"[compressed] {label}: compressing one group, T={T}, alloc {alloc}")
    cache = compressed_group(cfg, group, alloc, T)
    for tau in (0, 1):
        sc = cache["cells"][0][tau]["scales"]
        if sc is not None:
            say(f"[compressed] {label}: {'KV'[tau]} residual step median {np.median(sc):.2e}")
    h = J.jolt_load_cache(cache)
    inv = gen.rope_inv_freq_input(cfg.rope_base, d)
    scale = 1.0 / math.sqrt(d)
    Pi = rotation(cache["rotation_seed"], d)
    for layer in range(gs):
        q = gen.cfg_queries(cfg, 0, layer)[None]
        nb = J.jolt_decode_workspace_size([h], layer)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        qt = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).cuda()
        out = torch.full((1, cfg.H_q, d), float("nan"), dtype=torch.float32, device="cuda")
        J.jolt_decode_attention([h], layer, qt, [T], inv, scale, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()[0].astype(np.float64)
        assert np.isfinite(got).all()
        want = att.decode_layer(cache, layer, q[0].astype(np.float64), T, inv, scale, Pi,
                                heads=heads)
        for hh in heads:
            rows = slice(hh * Hg, (hh + 1) * Hg)
            r = float(np.linalg.norm(got[rows] - want[rows]) / np.linalg.norm(want[rows]))
            mx = float(np.max(np.abs(got[rows] - want[rows])))
            say(f"[compressed] {label} layer {layer} head {hh}: rel-L2 {r:.2e} max-abs {mx:.2e}")
            assert r <= 5e-3 and mx <= 2e-2, (layer, hh, r, mx)
