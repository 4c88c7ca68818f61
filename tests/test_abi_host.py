"""Host-side tests of the C-ABI library (no GPU needed).

* libjolt.so loads and exports every function include/jolt.h declares;
* jolt_make_rotation (the library's own SplitMix64 + Box-Muller + Householder
  QR) equals the oracle's rotation to 1e-12;
* argument validation: every rule in jolt.h returns its status code and a
  message before anything touches the GPU; the forced allocation-failure hook
  returns JOLT_E_OOM; batch == 0 is a no-op.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import compressed_cache_decode_jolt_amd as J
from compressed_cache_decode_jolt_amd import _jolt
from oracle.rotation import rotation

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(_jolt.LIB_PATH):
        from compressed_cache_decode_jolt_amd import build
        build.build(verbose=False)
    return J.lib()


def declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(jolt_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    lib = C.CDLL(_jolt.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_jolt.EXPORTS), "binding and header disagree"


@pytest.mark.parametrize("seed,d", [(0x4A4F4C54, 128), (0x4A4F4C54, 64), (1, 64), (2 ** 63 + 5, 128)])
def test_library_rotation_matches_oracle(seed, d):
    a = J.jolt_make_rotation(seed, d)
    b = rotation(seed, d)
    assert np.max(np.abs(a - b)) <= 1e-12
    assert np.max(np.abs(a.T @ a - np.eye(d))) < 1e-13


def base_cache(bits=(4, 2), T=64, d=64, H=2, H_q=4):
    g = np.random.default_rng(0)
    def cell(rT, rF, b):
        c = {"r_T": rT, "r_F": rF, "bits": b,
             "A": g.standard_normal((T, rT)).astype(np.float32),
             "B": g.standard_normal((d, rF)).astype(np.float32),
             "G": g.standard_normal((1, H, rT, rF)).astype(np.float32), "codes": None, "scales": None}
        if b:
            c["codes"] = g.integers(0, 256, (1, H, T, d * b // 8), dtype=np.uint8)
            c["scales"] = np.ones((1, H, T), np.float32)
        return c
    return {"T": T, "H": H, "H_q": H_q, "d": d, "n_layers": 1, "group_start": [0, 1],
            "factor_dtype": "f32", "rotation_seed": 1,
            "cells": [(cell(16, 16, bits[0]), cell(16, 16, bits[1]))]}


def expect(status, fn, *args, match=None):
    with pytest.raises(J.JoltError) as e:
        fn(*args)
    assert e.value.status == status, str(e.value)
    if match:
        assert re.search(match, str(e.value)), str(e.value)


def mutate(**kw):
    c = base_cache()
    for k, v in kw.items():
        if k.startswith("cell_"):
            c["cells"][0][0][k[5:]] = v
        else:
            c[k] = v
    return c


@pytest.mark.parametrize("cache,status,match", [
    (mutate(T=0), -1, "T=0"),
    (mutate(H_q=3), -1, "multiple"),
    (mutate(d=96), -2, "head_dim"),
    (mutate(H_q=2 * 17), -2, "query heads"),
    (mutate(group_start=[0, 2]), -1, "group_start"),
    (mutate(cell_bits=3), -1, "bits=3"),
    (mutate(cell_r_F=0), -1, "zero together"),
    (mutate(cell_r_T=65), -1, "r_T=65"),
    (mutate(cell_r_F=65), -1, "r_F=65"),
])
def test_load_validation(cache, status, match):
    expect(status, J.jolt_load_cache, cache, 0, match=match)


def test_codes_null_iff_bits_zero():
    c = base_cache(bits=(0, 2))
    c["cells"][0][0]["bits"] = 2          # bits > 0 but no codes
    expect(-1, J.jolt_load_cache, c, 0, match="codes/scales")


def test_forced_oom(monkeypatch):
    monkeypatch.setenv("JOLT_TEST_FAIL_ALLOC", "1")
    expect(-3, J.jolt_load_cache, base_cache(), 0, match="forced")


def test_error_message_is_thread_local_and_clears():
    expect(-1, J.jolt_load_cache, mutate(T=0), 0)
    assert "T=0" in J.jolt_last_error()
    J.jolt_make_rotation(1, 8)
    assert J.jolt_last_error() == ""


def test_empty_batch_is_noop():
    assert J.jolt_decode_workspace_size([], 0) == 0
    J.jolt_decode_attention([], 0, None, [], np.zeros(32, np.float32), 1.0, None, None, stream=0)


@pytest.mark.parametrize("args,status", [
    ((1, 8, 12, 128, 64), -1),     # n_q not a multiple of n_kv
    ((1, 8, 32, 96, 64), -2),      # unsupported d
    ((1, 8, 32, 128, 0), -1),      # T < 1
    ((-1, 8, 32, 128, 64), -1),    # batch < 0
])
def test_dense_validation(args, status):
    expect(status, J.jolt_dense_workspace_size, *args)


def test_dense_workspace_size_formula():
    n = J.jolt_dense_workspace_size(2, 8, 32, 128, 4096, split_tokens=256)
    assert n == 2 * 32 * (4096 // 256) * (4 + 128) * 4


def test_rope_domain_checked_before_launch():
    # positions above 2^20 or frequencies above 1 are rejected on the host
    assert J.jolt_decode_workspace_size([], 0) == 0
    expect(-1, J.jolt_debug_sincos, np.array([2.0 ** 21], np.float32), match="2\\^20")
    expect(-1, J.jolt_debug_sincos, np.array([1.0], np.float32), 3, match="variant")
    # the small-angle variant takes (position, inv_freq) pairs, inv_freq in [0, 1]
    expect(-1, J.jolt_debug_sincos, np.array([[5.0, 1.5]], np.float32), 2, match="inv_freq")
    expect(-1, J.jolt_debug_sincos, np.array([[2.0 ** 21, 0.5]], np.float32), 2, match="2\\^20")
    with pytest.raises(ValueError):
        J.jolt_debug_sincos(np.array([1.0, 0.5], np.float32), 2)


def test_long_context_rejected_at_load():
    expect(-2, J.jolt_load_cache, mutate(T=(1 << 20) + 1), 0, match="T=")


def test_compressor_entry_points_validate_before_device_work():
    """The compressor, grouping and quantiser entry points reject bad
    arguments with JOLT_E_INVALID before touching any device pointer (the
    pointers below are never dereferenced)."""
    L = J.lib()
    fake = C.c_void_p(0x1000)
    P = _jolt.jolt_flash_params(64, 16, 2, 0)
    out = (C.c_double * 200)()
    n2 = C.c_double()
    st = L.jolt_flash_spectra(fake, _jolt.JOLT_BF16, 1, 2, 128, 128, C.byref(_jolt.jolt_flash_params(0, 16, 2, 0)),
                              out, out, C.addressof(n2), None)
    assert st == -1 and b"flash params" in L.jolt_last_error()
    st = L.jolt_flash_spectra(fake, _jolt.JOLT_BF16, 1, 2, 128, 129 + 127, C.byref(P), out, out,
                              C.addressof(n2), None)
    assert st == -1 and b"shape" in L.jolt_last_error()
    st = L.jolt_flash_spectra(fake, _jolt.JOLT_BF16, 1, 2, 128, 128, C.byref(P), None, out,
                              C.addressof(n2), None)
    assert st == -1
    # ranks: r_T above q_cap, r_T = 0 with r_F > 0, bits 3
    for rT, rF, b in [(96, 32, 4), (0, 16, 0), (32, 16, 3)]:
        st = L.jolt_flash_compress_cell(fake, _jolt.JOLT_BF16, 1, 2, 128, 128, C.byref(P), rT, rF, b,
                                        C.c_uint64(1), _jolt.JOLT_BF16, fake, fake, fake, fake, fake, None)
        assert st == -1, (rT, rF, b)
    ks = (C.c_void_p * 2)(0x1000, 0x2000)
    starts = (C.c_int32 * 3)()
    ng = C.c_int32()
    st = L.jolt_flash_layer_groups(ks, ks, _jolt.JOLT_BF16, 2, 2, 128, 128, C.byref(P),
                                   C.c_double(float("nan")), 0, starts, C.byref(ng), None, None)
    assert st == -1 and b"bad arguments" in L.jolt_last_error()
    st = L.jolt_quantize_rows(fake, 4, 128, 3, fake, fake, None)
    assert st == -1 and b"bits=3" in L.jolt_last_error()
