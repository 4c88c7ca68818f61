"""GPU parity over a seeded sweep of random shapes: lengths (ragged, below a
tile, several splits), head groupings H_grp in {1, 2, 4, 8, 16}, ranks and
residual bits of every launch class, batches that mix classes and lengths,
and explicit split sizes.  Each case compares the HIP path (automatic kernel
choice, through the C ABI) with the oracle at the tolerances of the kernel
that ran: the MFMA kernel for bf16 caches with d = 128, the float32 kernel
otherwise."""
import numpy as np
import pytest

import compressed_cache_decode_jolt_amd as J
from oracle import attention as att
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BITS = [0, 2, 4, 8]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    J.lib()


def _rank(r, T, H, d, lo, hi):
    """A rank in [lo, hi] (0 allowed) within the ABI's r_T <= min(T, H d)."""
    r_T = int(r.integers(lo, hi + 1))
    r_T = min(r_T, T, H * d)
    if r_T == 0:
        return 0, 0
    return r_T, int(r.integers(1, d + 1))


def _case(seed):
    r = np.random.default_rng([0x5EED, seed])
    wide = r.random() < 0.3                        # key ranks above 256
    d = 128 if wide or r.random() < 0.85 else 64
    H = 4 if wide else int(r.choice([1, 2, 4]))
    Hg = int(r.choice([1, 2, 4, 8, 16]))
    B = int(r.choice([1, 1, 2, 3]))
    spec = []
    for b in range(B):
        T = int(r.choice([513, 777, 1200] if wide else [1, 15, 17, 100, 129, 300, 513, 777, 1200]))
        if wide:
            kr = _rank(r, T, H, d, 257, 512)
            vr = _rank(r, T, H, d, 0, 256)
        else:
            kr = _rank(r, T, H, d, 0, 256)
            vr = _rank(r, T, H, d, 0, 512)
        bk, bv = int(r.choice(BITS)), int(r.choice(BITS))
        spec.append((T, (kr[0], kr[1], bk), (vr[0], vr[1], bv)))
    split = int(r.choice([0, 0, 128, 256, 640]))
    return d, H, H * Hg, spec, split


@pytest.mark.parametrize("seed", range(48))
def test_random_shape(seed):
    d, H, H_q, spec, split = _case(seed)
    caches = [gen.small_cache(500 + 10 * seed + i, T, H, H_q, d, [(aK, aV)], [1])
              for i, (T, aK, aV) in enumerate(spec)]
    inv = gen.rope_inv_freq_input(5e5 if d == 128 else 1e4, d)
    q = np.stack([gen.queries(501 + seed, i, 0, H_q, d, "bf16") for i in range(len(spec))])
    q_pos = [T for T, _, _ in spec]
    hs = [J.jolt_load_cache(c) for c in caches]
    qt = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).cuda()
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    nb = J.jolt_decode_workspace_size(hs, 0, split_tokens=split)
    ws = torch.zeros(max(nb, 1), dtype=torch.uint8, device="cuda")
    J.jolt_decode_attention(hs, 0, qt, q_pos, inv, 0.088, out, ws, split_tokens=split)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = att.decode_attention(caches, 0, q.astype(np.float64), q_pos, inv, 0.088)
    mfma = d == 128   # bf16 caches: the automatic choice takes the MFMA kernel when it fits
    for b in range(len(spec)):
        norm = np.linalg.norm(want[b])
        if norm == 0:
            assert np.all(got[b] == 0), (seed, b, spec[b])
            continue
        rel = float(np.linalg.norm(got[b] - want[b]) / norm)
        mx = float(np.max(np.abs(got[b] - want[b])))
        if mfma:
            assert rel <= 5e-3 and mx <= 2e-2, (seed, b, spec[b], split, rel, mx)
        else:
            assert rel <= 1e-5, (seed, b, spec[b], split, rel)
