"""Pins for oracle.grouping (alignment-based layer grouping).

* alignment is 1 for a layer with itself, symmetric, in [0, 1], and 0 for
  orthogonal subspaces (exact constructions);
* on the synthetic generator's caches, whose layers share one token basis
  within a generated group and draw independent bases across groups, the
  grouping recovers exactly the generated groups;
* identical layers form one run; max_group splits long runs;
* the threshold decides: tau above every alignment gives singletons.
"""
import numpy as np
import pytest

from oracle import grouping as gr
from workloads import gen


def layers_from_groups(n_groups, gs=4, H=2, T=512, d=32, seed=0):
    out = []
    for g in range(n_groups):
        XK = gen.kv_tensor((91, seed, g, 0), gs, H, T, d, 1.0, True, 1, rank=16)
        XV = gen.kv_tensor((91, seed, g, 1), gs, H, T, d, 0.6, False, 0, rank=16)
        out += [(XK[l], XV[l]) for l in range(gs)]
    return out


def test_alignment_closed_forms():
    g = np.random.default_rng(0)
    Q, _ = np.linalg.qr(g.standard_normal((100, 20)))
    A, B = Q[:, :10], Q[:, 10:]
    assert gr.alignment(A, A) == pytest.approx(1.0, abs=1e-12)
    assert gr.alignment(A, B) == pytest.approx(0.0, abs=1e-12)
    C, _ = np.linalg.qr(g.standard_normal((100, 10)))
    assert gr.alignment(A, C) == pytest.approx(gr.alignment(C, A), rel=1e-12)
    assert 0.0 <= gr.alignment(A, C) <= 1.0
    # half of the subspace shared: alignment 1/2
    D = np.concatenate([A[:, :5], B[:, :5]], axis=1)
    assert gr.alignment(A, D) == pytest.approx(0.5, abs=1e-12)


def test_recovers_the_generated_groups():
    layers = layers_from_groups(3)
    starts, a = gr.align_groups(layers, 8, 0.5)
    assert starts == [0, 4, 8, 12]
    within = [a[l] for l in range(11) if (l + 1) % 4]
    across = [a[3], a[7]]
    assert min(within) > 0.55 and max(across) < 0.1


def test_identical_layers_one_run_and_max_group():
    XK = gen.kv_tensor((90, 0, 0, 0), 1, 2, 256, 32, 1.0, True, 1, rank=12)[0]
    XV = gen.kv_tensor((90, 0, 0, 1), 1, 2, 256, 32, 0.5, False, 0, rank=12)[0]
    layers = [(XK, XV)] * 7
    starts, a = gr.align_groups(layers, 8, 0.5)
    assert starts == [0, 7] and np.allclose(a, 1.0, atol=1e-9)
    starts, _ = gr.align_groups(layers, 8, 0.5, max_group=3)
    assert starts == [0, 3, 6, 7]
    starts, _ = gr.align_groups(layers, 8, 1.5)
    assert starts == list(range(8))
