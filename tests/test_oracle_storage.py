"""Pin oracle.storage rounding against torch's float32 -> bfloat16 conversion
(a library routine) on random values and on hand-made ties."""
import numpy as np
import torch

from oracle.storage import round_bf16, round_f32


def torch_bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_random_values_match_torch():
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(100000) * 10.0 ** g.integers(-30, 30, 100000),
                        g.standard_normal(1000) * 1e-40])
    assert np.array_equal(round_bf16(x), torch_bf16(x.astype(np.float32)))


def test_ties_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: even mantissa wins (1)
    assert round_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert round_bf16(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2.0 ** -6)


def test_f32_rounding_matches_torch():
    x = np.random.default_rng(2).standard_normal(1000)
    want = torch.from_numpy(x).to(torch.float32).to(torch.float64).numpy()
    assert np.array_equal(round_f32(x), want)
