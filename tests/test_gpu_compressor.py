"""GPU parity of the compressor (FlashJoLT, through the C ABI) against the
oracle's FlashJoLT (oracle.flash), which follows the same steps in numpy
float64 from the same seeded Gaussian test matrix.

* quantiser + packer on the oracle's rotated rows: codes and scales
  byte-identical to oracle.quant (every width, d = 64 and 128, zero rows,
  rows with exact rounding ties);
* spectra: the q_cap token energies, the synthetic tail entry, the feature
  energies and ||X||^2 within 1e-9 relative;
* compressed cells: the stored reconstruction A_s G_s B_s^T (independent of
  the factors' signs) within 1e-6 relative Frobenius, residual scales within
  one float32 ulp, residual codes identical except at rounding ties
  (counted: at most 1e-4 of them, each one level off);
* the GPU-compressed cache decodes on the GPU like the oracle decodes it.
"""
import math
import time

import numpy as np
import pytest

import compressed_cache_decode_jolt_amd as J
from oracle import attention as att
from oracle import flash
from oracle.quant import pack, quantize_rows
from oracle.rotation import rotation
from workloads import gen, get_config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    J.lib()


# -------------------------------------------------------------- quantiser --
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_quantize_rows_byte_identical(bits, d):
    g = np.random.default_rng(bits * 10 + d)
    R = g.standard_normal((4000, d)) * np.exp(g.standard_normal((4000, 1)))
    R[7] = 0.0                                       # delta = 0
    L = (1 << bits) - 1
    Pi = rotation(3, d)
    rows = R @ Pi                                    # the oracle's rotated rows
    # rows whose entries sit exactly on rounding ties of their own grid
    for row in range(10, 20):
        m = 3.0
        delta = np.float64(np.float32(2 * m / L))
        k = g.integers(0, L, size=d).astype(np.float64)
        rows[row] = (k + 0.5 - L / 2.0) * delta
        rows[row, 0] = m
    want_c, want_s = quantize_rows(rows, bits)
    got_c, got_s = J.jolt_quantize_rows(torch.from_numpy(rows).cuda(), bits)
    torch.cuda.synchronize()
    assert np.array_equal(got_c.cpu().numpy(), pack(want_c, bits))
    assert np.array_equal(got_s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))


# ------------------------------------------------------------ compressor --
def cell_input(cfg_idx, tau, T=None, dtype="bf16"):
    cfg = get_config(cfg_idx)
    X = gen.kv_group(cfg, 0, 0, tau, T=T)
    if dtype == "bf16":
        X = gen.to_bf16_values(X).astype(np.float64)
    else:
        X = X.astype(np.float32).astype(np.float64)
    t = torch.from_numpy(X.astype(np.float32)).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    return cfg, X, t.cuda().contiguous()


FLASH = dict(oversample=16, power_iters=2, sketch_seed=11)


@pytest.mark.parametrize("cfg_idx,tau,q_cap,dtype", [(1, 0, 64, "bf16"), (1, 1, 96, "bf16"),
                                                     (0, 1, 32, "f32")])
def test_spectra_match_oracle(cfg_idx, tau, q_cap, dtype):
    cfg, X, Xt = cell_input(cfg_idx, tau, dtype=dtype)
    sT2, sF2, n2 = J.jolt_flash_spectra(Xt, q_cap, **FLASH)
    wT2, wF2, wn2 = flash.flash_spectra(X, q_cap, **FLASH)
    assert n2 == pytest.approx(wn2, rel=1e-12)
    assert np.allclose(sT2, wT2, rtol=1e-9, atol=1e-12 * wn2)
    assert np.allclose(sF2, wF2, rtol=1e-9, atol=1e-12 * wn2)


def stored_recon(cell):
    A, B, G = (cell[k].astype(np.float64) for k in ("A", "B", "G"))
    return np.einsum("tr,lhrs,fs->lhtf", A, G, B, optimize=True)


CELLS = [(1, 0, (48, 64, 4), 64, "bf16"), (1, 1, (64, 64, 4), 64, "bf16"),
         (1, 1, (96, 128, 8), 96, "bf16"), (1, 0, (32, 32, 2), 48, "bf16"),
         (1, 0, (0, 0, 8), 16, "bf16"), (1, 1, (64, 64, 0), 64, "bf16"),
         (0, 0, (32, 16, 4), 32, "f32")]


@pytest.mark.parametrize("cfg_idx,tau,alloc,q_cap,dtype", CELLS,
                         ids=[f"cfg{c[0]}-{'KV'[c[1]]}-{c[2]}" for c in CELLS])
def test_compressed_cell_matches_oracle(cfg_idx, tau, alloc, q_cap, dtype):
    cfg, X, Xt = cell_input(cfg_idx, tau, dtype=dtype)
    r_T, r_F, bits = alloc
    t0 = time.perf_counter()
    got = J.jolt_flash_compress_cell(Xt, r_T, r_F, bits, q_cap, 0x4A4F4C54, dtype, **FLASH)
    t_gpu = time.perf_counter() - t0
    Pi = rotation(0x4A4F4C54, cfg.d)
    t0 = time.perf_counter()
    want = flash.flash_compress_cell(X, r_T, r_F, bits, dtype, Pi, q_cap, **FLASH)
    t_ora = time.perf_counter() - t0
    print(f"compress {cfg.name} {'KV'[tau]} {alloc}: GPU {t_gpu:.3f} s, oracle {t_ora:.3f} s")
    if r_T:
        a, b = stored_recon(got), stored_recon(want)
        assert np.linalg.norm(a - b) <= 1e-6 * np.linalg.norm(b)
    if bits:
        gs, ws = got["scales"], want["scales"]
        ulp = np.abs(gs.view(np.int32).astype(np.int64) - ws.view(np.int32).astype(np.int64))
        assert ulp.max() <= 1
        from oracle.quant import unpack
        gc = unpack(got["codes"], bits, cfg.d).astype(np.int64)
        wc = unpack(want["codes"], bits, cfg.d).astype(np.int64)
        diff = gc != wc
        print(f"  codes differing (rounding ties): {int(diff.sum())} of {diff.size}")
        assert diff.mean() <= 1e-4 and np.abs(gc - wc).max() <= 1


def test_gpu_compressed_cache_decodes_like_oracle():
    """Compress the 4K-token layer on the GPU at its 3x allocation, load it,
    decode on the GPU and compare with the oracle's decode of that cache."""
    import json, os
    cfg = get_config(1)
    alloc = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "allocations.json")))
    (aK, aV), = alloc["1"]["tables"]["3x"]["groups"]
    cells = []
    for tau, a in ((0, aK), (1, aV)):
        _, _, Xt = cell_input(1, tau)
        cells.append(J.jolt_flash_compress_cell(Xt, *a, 96, 0x4A4F4C54, "bf16", **FLASH))
    cache = {"T": cfg.T, "H": cfg.H, "H_q": cfg.H_q, "d": cfg.d, "n_layers": 1,
             "group_start": [0, 1], "factor_dtype": "bf16", "rotation_seed": 0x4A4F4C54,
             "cells": [tuple(cells)]}
    h = J.jolt_load_cache(cache)
    inv = gen.rope_inv_freq_input(cfg.rope_base, cfg.d)
    q = gen.cfg_queries(cfg, 0, 0)[None]
    qt = torch.from_numpy(q).to(torch.bfloat16).cuda()
    out = torch.empty((1, cfg.H_q, cfg.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(J.jolt_decode_workspace_size([h], 0), dtype=torch.uint8, device="cuda")
    J.jolt_decode_attention([h], 0, qt, [cfg.T], inv, 1 / math.sqrt(cfg.d), out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = att.decode_attention([cache], 0, q.astype(np.float64), [cfg.T], inv, 1 / math.sqrt(cfg.d))
    r = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    assert r <= 5e-3 and float(np.max(np.abs(got - want))) <= 2e-2


@pytest.mark.timeout(600)
def test_gpu_pipeline_matches_oracle_pipeline():
    """Spectra -> native allocator -> cells on the GPU (compressor.compress_cache)
    against the oracle's FlashJoLT pipeline at 3x on two layer groups of the
    64K stack's shape (T shortened to 4096): the same allocation table, stored
    reconstructions within 1e-6, and the GPU decode of the GPU-built cache
    against the oracle's decode of it."""
    from compressed_cache_decode_jolt_amd.compressor import compress_cache
    from oracle.compress import budget_for
    cfg = get_config(2)
    T, ng = 4096, 2
    host, dev = [], []
    for g in range(ng):
        pair = [gen.to_bf16_values(gen.kv_group(cfg, 0, g, tau, T=T)).astype(np.float64)
                for tau in (0, 1)]
        host.append(tuple(pair))
        dev.append(tuple(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda()
                         for x in pair))
    starts = [0, 4, 8]
    budget = budget_for(3.0, 8, cfg.H, cfg.d, T)
    t0 = time.perf_counter()
    cache, alloc = compress_cache(dev, cfg.H_q, starts, budget=budget, q_cap=128, **FLASH)
    t_gpu = time.perf_counter() - t0
    t0 = time.perf_counter()
    want_cache, want_alloc = flash.flash_compress(host, budget, "bf16", 0x4A4F4C54, cfg.H_q, starts,
                                                  128, **FLASH)
    t_ora = time.perf_counter() - t0
    print(f"pipeline (2 groups x 4 layers, T={T}): GPU {t_gpu:.2f} s, oracle {t_ora:.2f} s; "
          f"allocation {alloc}")
    assert [tuple(map(tuple, a)) for a in alloc] == [tuple(map(tuple, a)) for a in want_alloc]
    for g in range(ng):
        for tau in (0, 1):
            a, b = cache["cells"][g][tau], want_cache["cells"][g][tau]
            if a["r_T"]:
                ra, rb = stored_recon(a), stored_recon(b)
                assert np.linalg.norm(ra - rb) <= 1e-6 * np.linalg.norm(rb)
    h = J.jolt_load_cache(cache)
    inv = gen.rope_inv_freq_input(cfg.rope_base, cfg.d)
    for layer in (0, 5):
        q = gen.cfg_queries(cfg, 0, layer)[None]
        qt = torch.from_numpy(q).to(torch.bfloat16).cuda()
        out = torch.empty((1, cfg.H_q, cfg.d), dtype=torch.float32, device="cuda")
        ws = torch.empty(J.jolt_decode_workspace_size([h], layer), dtype=torch.uint8, device="cuda")
        J.jolt_decode_attention([h], layer, qt, [T], inv, 1 / math.sqrt(cfg.d), out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        want = att.decode_attention([cache], layer, q.astype(np.float64), [T], inv,
                                    1 / math.sqrt(cfg.d))
        assert float(np.linalg.norm(got - want) / np.linalg.norm(want)) <= 5e-3
        assert float(np.max(np.abs(got - want))) <= 2e-2
