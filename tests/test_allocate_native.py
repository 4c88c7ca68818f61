"""The library's native allocator (jolt_allocate, host C++, no GPU) against
the oracle's allocator (oracle.allocate) on the same spectra: identical
(r_T, r_F, bits) for every cell and the same multiplier, over exhaustive and
coordinate-wise cells, caps, FlashJoLT spectra with the synthetic tail entry,
and budgets from loose to tight."""
import numpy as np
import pytest

import compressed_cache_decode_jolt_amd as J
from oracle import allocate as al
from oracle.compress import budget_for, cell_stats
from oracle.flash import flash_spectra
from workloads import gen


def as_native(st, cap=None):
    return {"T": st.T, "d": st.d, "group_size": st.group_size, "H": st.H,
            "factor_bytes": st.factor_bytes, "sT2": st.sT2, "sF2": st.sF2, "norm2": st.norm2,
            "cap": cap or 0}


def cells_for(seed, T, d, gs, H, rank=24, flash_q=None):
    out = []
    for tau, alpha in ((0, 1.0), (1, 0.3)):
        X = gen.kv_tensor((92, seed, 0, tau), gs, H, T, d, alpha, tau == 0, 2, rank=rank)
        if flash_q:
            sT2, sF2, n2 = flash_spectra(X, flash_q, 16, 2, seed)
            out.append(al.CellStats(T=T, d=d, group_size=gs, H=H, factor_bytes=2, sT2=sT2,
                                    sF2=sF2, norm2=n2, cap=flash_q))
        else:
            out.append(cell_stats(X, 2))
    return out


CASES = [  # (seed, T, d, gs, H, flash q_cap)
    (0, 64, 32, 1, 2, None),       # tiny grids, exhaustive
    (1, 256, 64, 2, 2, None),
    (2, 1024, 128, 1, 8, None),    # grid of 65 x 9 x 4: exhaustive
    (3, 2048, 128, 2, 8, None),    # grid above 1e5 points: coordinate-wise
    (4, 2048, 128, 2, 4, 64),      # FlashJoLT spectra, rank cap 64
]


@pytest.mark.parametrize("seed,T,d,gs,H,fq", CASES)
@pytest.mark.parametrize("ratio", [1.5, 2.0, 3.0, 5.0, 12.0])
def test_native_allocator_equals_oracle(seed, T, d, gs, H, fq, ratio):
    cells = cells_for(seed, T, d, gs, H, flash_q=fq)
    if fq:
        for c in cells:
            c.cap = fq
    budget = budget_for(ratio, gs, H, d, T)
    want, lam_w = al.allocate(cells, budget)
    got, lam_g = J.jolt_allocate([as_native(c, c.cap) for c in cells], budget)
    assert [tuple(x) for x in got] == [tuple(x) for x in want]
    assert lam_g == pytest.approx(lam_w, rel=1e-9, abs=0)


def test_native_allocator_rejects_infeasible_budget():
    cells = cells_for(0, 64, 32, 1, 2)
    with pytest.raises(J.JoltError):
        J.jolt_allocate([as_native(c) for c in cells], -1.0)
