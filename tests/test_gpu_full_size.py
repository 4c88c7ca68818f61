"""GPU parity at the workloads' full sizes, on sampled outputs.

Each case builds the workload's caches at full T, heads, head dim and
batch (per-sequence allocations where the workload allocates each sequence
on its own), restricted to a few whole layer groups, and runs
jolt_decode_attention the way bench.py does (automatic kernel and split).
The oracle then decodes a sample of (sequence, KV head) pairs of the
checked layers one by one and the corresponding query-head rows are
compared:
  * MFMA path (bf16 factors, d = 128): rel-L2 <= 5e-3 and max-abs <= 2e-2;
  * float32-arithmetic path (shapes the MFMA kernel does not take):
    rel-L2 <= 1e-5 and max-abs <= 1e-4.
The stored values are synthetic (random factors of the allocated ranks,
uniform codes, scales of the workload's magnitude): the decode computes
the same function of whatever is stored.
"""
import json
import math
import os
import sys

import numpy as np
import pytest

import compressed_cache_decode_jolt_amd as J
from oracle import attention as att
from oracle.rotation import rotation
from workloads import gen, get_config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ALLOC = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                    "allocations.json")))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    J.lib()


def alloc_of(cfg, ratio, seq):
    t = ALLOC[str(cfg.idx)]["tables"]
    if "fixed" in t:
        key = "fixed"
    else:
        key = f"{ratio}/seq{seq}" if f"{ratio}/seq{seq}" in t else ratio
    return [tuple(map(tuple, g)) for g in t[key]["groups"]]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# (workload, budget, layer groups built, sequences sampled, KV heads sampled)
CASES = [
    (2, "3x", [0, 6], [0], [0, 5]),        # K (192,128,4) and (32,128,8)
    (2, "2x", [0, 4], [0], [2, 7]),        # 8-bit keys, 8- and 4-bit values
    (2, "5x", [1, 7], [0], [1, 6]),        # 2-bit values
    (3, "2.5x", [4, 9], [0, 1, 3], [0, 7]),  # batch 4, per-sequence bits, 8 q heads per KV head
    (4, "fixed", [0], [0, 15], [0, 31]),   # MHA batch 16, value rank 512 (4-wave class)
    (4, "fixed", [7], [0, 15], [3, 30]),   # key rank 512: the float32 path
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg_idx,ratio,groups,seqs,heads", CASES,
                         ids=[f"cfg{c[0]}-{c[1]}-g{'-'.join(map(str, c[2]))}" for c in CASES])
def test_full_size_sampled(cfg_idx, ratio, groups, seqs, heads):
    cfg = get_config(cfg_idx)
    B, gs, d = cfg.batch, cfg.group_size, cfg.d
    say(f"[full-size] {cfg.name} {ratio} groups {groups}: building {B} caches, T={cfg.T}")
    caches = []
    for s in range(B):
        al = alloc_of(cfg, ratio, s)
        caches.append(gen.synthetic_cache(cfg, [al[g] for g in groups], seq=s,
                                          layers=len(groups) * gs))
    handles = [J.jolt_load_cache(c) for c in caches]
    inv = gen.rope_inv_freq_input(cfg.rope_base, d)
    scale = 1.0 / math.sqrt(d)
    Pi = rotation(caches[0]["rotation_seed"], d)
    Hg = cfg.H_q // cfg.H
    for gi in range(len(groups)):
        for layer in (gi * gs, gi * gs + gs - 1):
            q = np.stack([gen.cfg_queries(cfg, s, layer) for s in range(B)])
            try:
                J.jolt_decode_workspace_size(handles, layer, kernel=J.KERNEL_MFMA)
                rt, at = 5e-3, 2e-2
                path = "mfma"
            except J.JoltError:
                rt, at = 1e-5, 1e-4
                path = "f32"
            nb = J.jolt_decode_workspace_size(handles, layer)
            ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
            qt = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).cuda()
            out = torch.full((B, cfg.H_q, d), float("nan"), dtype=torch.float32, device="cuda")
            J.jolt_decode_attention(handles, layer, qt, [cfg.T] * B, inv, scale, out, ws)
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
            assert np.isfinite(got).all()
            for s in seqs:
                want = att.decode_layer(caches[s], layer, q[s].astype(np.float64), cfg.T, inv,
                                        scale, Pi, heads=heads)
                for h in heads:
                    rows = slice(h * Hg, (h + 1) * Hg)
                    r = float(np.linalg.norm(got[s, rows] - want[rows]) /
                              np.linalg.norm(want[rows]))
                    mx = float(np.max(np.abs(got[s, rows] - want[rows])))
                    say(f"[full-size] {cfg.name} layer {layer} seq {s} head {h} ({path}): "
                        f"rel-L2 {r:.2e} max-abs {mx:.2e}")
                    assert r <= rt and mx <= at, (layer, s, h, r, mx)
