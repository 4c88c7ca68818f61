"""Pins for oracle.accounting against the byte figures the JoLT pages print
(tests/golden/kv_bytes.json, each entry cited)."""
import json
import os

import numpy as np
import pytest

from oracle.accounting import cache_bytes, cell_bytes, dense_kv_bytes

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_bytes.json")))


@pytest.mark.parametrize("e", GOLD["entries"], ids=lambda e: e["what"])
def test_dense_kv_bytes_against_pages(e):
    n = dense_kv_bytes(e["layers"], e["kv_heads"], e["head_dim"], e["seq_len"], e["dtype_bytes"])
    if "exact" in e:
        assert n == e["exact"]
    if "approx_gib" in e:
        assert n / 2 ** 30 == pytest.approx(e["approx_gib"], rel=1e-12)
    if "approx_kib" in e:
        assert n / 2 ** 10 == pytest.approx(e["approx_kib"], rel=1e-12)
    if "approx_mib" in e:
        assert round(n / 2 ** 20, 2) == e["approx_mib"]
    if "approx_mb" in e:
        assert round(n / 1e6, 1) == e["approx_mb"]
    if "min_gib" in e:
        assert n / 2 ** 30 > e["min_gib"]


def test_gqa_cuts_exactly_by_head_ratio():
    # the sarnas.ru post: GQA (8 KV heads instead of 64) cuts the cache exactly 8x
    assert dense_kv_bytes(80, 64, 128, 1) == 8 * dense_kv_bytes(80, 8, 128, 1)


def test_cell_bytes_parts():
    # factors only (b=0), then one residual row per (layer, head, token)
    T, d, gs, H = 100, 64, 3, 5
    assert cell_bytes(T, d, gs, H, 0, 0, 0, 2) == 0
    assert cell_bytes(T, d, gs, H, 16, 32, 0, 2) == 2 * (T * 16 + d * 32 + gs * H * 16 * 32)
    for b in (2, 4, 8):
        assert cell_bytes(T, d, gs, H, 0, 0, b, 2) == gs * H * T * (d * b // 8 + 4)
    assert cell_bytes(T, d, gs, H, 16, 16, 4, 4) == \
        cell_bytes(T, d, gs, H, 16, 16, 0, 4) + cell_bytes(T, d, gs, H, 0, 0, 4, 4)


def test_cache_bytes_sums_cells():
    cell = lambda rT, rF, b: {"r_T": rT, "r_F": rF, "bits": b}  # noqa: E731
    cache = {"T": 64, "d": 32, "H": 2, "factor_dtype": "bf16", "group_start": [0, 2, 3],
             "cells": [(cell(16, 16, 2), cell(32, 16, 0)), (cell(0, 0, 8), cell(16, 32, 4))]}
    want = (cell_bytes(64, 32, 2, 2, 16, 16, 2, 2) + cell_bytes(64, 32, 2, 2, 32, 16, 0, 2)
            + cell_bytes(64, 32, 1, 2, 0, 0, 8, 2) + cell_bytes(64, 32, 1, 2, 16, 32, 4, 2))
    assert cache_bytes(cache) == want


def stored_bytes(cache):
    """Bytes of the arrays oracle.compress.compress actually stores, each in
    its storage dtype: A, B, G at the factor dtype's size per element, the
    packed codes as uint8 and one float32 scale per quantised row."""
    fb = {"bf16": 2, "f32": 4}[cache["factor_dtype"]]
    total = 0
    for pair in cache["cells"]:
        for cell in pair:
            total += fb * (cell["A"].size + cell["B"].size + cell["G"].size)
            if cell["codes"] is not None:
                assert cell["codes"].dtype == np.uint8 and cell["scales"].dtype == np.float32
                total += cell["codes"].nbytes + cell["scales"].nbytes
    return total


@pytest.mark.parametrize("factor_dtype", ["bf16", "f32"])
def test_cache_bytes_equals_stored_arrays(factor_dtype):
    """O10 against what the compressor really stores (several layers per
    group, several heads, every residual width, a rank-0 cell), not against
    a restatement of the formula."""
    from oracle.compress import compress
    from workloads import gen

    T, d, H = 48, 32, 3
    sizes = [2, 1, 3]
    alloc = [((16, 16, 0), (32, 16, 2)), ((0, 0, 4), (16, 32, 8)), ((32, 32, 8), (0, 0, 0))]
    groups = []
    for g, gs in enumerate(sizes):
        groups.append(tuple(gen.kv_tensor((97, 0, g, tau), gs, H, T, d, 1.0 - 0.6 * tau, tau == 0, 1,
                                          rank=8) for tau in (0, 1)))
    starts = list(np.cumsum([0] + sizes))
    cache = compress(groups, alloc, factor_dtype, 11, 2 * H, starts)
    assert stored_bytes(cache) == cache_bytes(cache)
    # and per cell: the stored shapes are the ones O10 counts
    for (gK, gV), gs, (aK, aV) in zip(cache["cells"], sizes, alloc):
        for cell, (rT, rF, b) in ((gK, aK), (gV, aV)):
            assert cell["A"].shape == (T, rT) and cell["B"].shape == (d, rF)
            assert cell["G"].shape == (gs, H, rT, rF)
            if b:
                assert cell["codes"].shape == (gs, H, T, d * b // 8)
                assert cell["scales"].shape == (gs, H, T)
            else:
                assert cell["codes"] is None and cell["scales"] is None
