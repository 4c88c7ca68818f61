"""Workload shapes.

Five decode workloads, named by what they model:

* ``tiny-fp32``      one layer, 2 KV heads, 8 query heads, d=64, T=256, fp32
                     everywhere, fixed ranks (32, 16) and 4-bit residual.
* ``llama3-8b-layer`` one Llama-3.1-8B-shaped layer (8 KV / 32 query heads,
                     d=128) at T=4096, bf16, allocator at a 3x byte budget.
* ``llama3-8b-64k``  the full 32-layer Llama-3.1-8B stack (8 groups of 4
                     layers) at T=65536, allocator at 2/3/4/5x.
* ``llama3-70b``     80 layers (20 groups of 4), 8 KV / 64 query heads,
                     T=32768, 4 independent sequences, allocator at 2.5x.
* ``mha-7b``         32 layers (8 groups), 32 KV = 32 query heads (no GQA),
                     T=8192, 16 sequences, a fixed rank/bit schedule.

The KV-cache shapes follow the models the JoLT pages evaluate (LLaMA-3.1-8B
RULER at 64K, the 70B byte arithmetic, an MHA LLaMA-2-like model); the data is
synthetic (see ``gen.py``).
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

ROTATION_SEED = 0x4A4F4C54  # "JOLT"


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    batch: int            # independent sequences per decode step
    n_layers: int
    group_size: int       # consecutive layers per layer group
    H: int                # KV heads
    H_q: int              # query heads
    d: int                # head dim
    T: int                # cached tokens per sequence
    rope_base: float
    factor_dtype: str     # "f32" or "bf16"
    q_dtype: str          # "f32" or "bf16"
    n_out: int            # key outlier channels (x8)
    alpha_K: float = 1.0
    alpha_V: float = 0.3
    budgets: Tuple[float, ...] = ()
    fixed: Optional[Tuple[int, int, int]] = None   # (r_T, r_F, bits) for every cell
    schedule: Optional[str] = None                 # named fixed per-group schedule

    @property
    def n_groups(self):
        return self.n_layers // self.group_size

    @property
    def H_grp(self):
        return self.H_q // self.H

    @property
    def factor_bytes(self):
        return 4 if self.factor_dtype == "f32" else 2

    def group_start(self):
        return [g * self.group_size for g in range(self.n_groups + 1)]

    def alpha(self, tau, group):
        """Spectral decay exponent of the synthetic basis for (K/V, group).

        Multi-group workloads ramp the exponent linearly over groups
        (0.8x .. 1.2x) so that groups differ in compressibility.
        """
        a = self.alpha_K if tau == 0 else self.alpha_V
        if self.n_groups > 1:
            a = a * (0.8 + 0.4 * group / (self.n_groups - 1))
        return a


CONFIGS = {
    0: Config(0, "tiny-fp32", batch=1, n_layers=1, group_size=1, H=2, H_q=8, d=64,
              T=256, rope_base=1e4, factor_dtype="f32", q_dtype="f32", n_out=2,
              fixed=(32, 16, 4)),
    1: Config(1, "llama3-8b-layer", batch=1, n_layers=1, group_size=1, H=8, H_q=32,
              d=128, T=4096, rope_base=5e5, factor_dtype="bf16", q_dtype="bf16",
              n_out=4, budgets=(3.0,)),
    2: Config(2, "llama3-8b-64k", batch=1, n_layers=32, group_size=4, H=8, H_q=32,
              d=128, T=65536, rope_base=5e5, factor_dtype="bf16", q_dtype="bf16",
              n_out=4, budgets=(2.0, 3.0, 4.0, 5.0)),
    3: Config(3, "llama3-70b", batch=4, n_layers=80, group_size=4, H=8, H_q=64,
              d=128, T=32768, rope_base=5e5, factor_dtype="bf16", q_dtype="bf16",
              n_out=4, alpha_V=0.2, budgets=(2.5,)),
    4: Config(4, "mha-7b", batch=16, n_layers=32, group_size=4, H=32, H_q=32,
              d=128, T=8192, rope_base=1e4, factor_dtype="bf16", q_dtype="bf16",
              n_out=4, schedule="mha-7b"),
}


def get_config(key):
    if isinstance(key, int):
        return CONFIGS[key]
    for c in CONFIGS.values():
        if c.name == key:
            return c
    raise KeyError(key)


def mha7b_schedule(group):
    """Fixed (r_T, r_F, bits) per group for the MHA workload: ((K), (V))."""
    kf = [32, 48, 64, 80, 96, 32, 64, 96]
    kb = [0, 2, 4, 8, 0, 2, 4, 8]
    vf = [96, 80, 64, 48, 32, 96, 64, 32]
    vb = [4, 8, 0, 2, 4, 8, 0, 2]
    return ((64 * (group + 1), kf[group], kb[group]),
            (64 * (8 - group), vf[group], vb[group]))
