"""The five benchmark workloads of the HSTU layer, as plain size records.

Shapes follow the model the DLRMv4 page describes ("DLRMv4 Brings
Sequence-Based Recommendation Training to MLPerf", section "HSTU
Hyperparameters", Table 5: d_model 512, 4 heads of 128, sequences up to 4096,
bf16) and widen it to a small fp32 case, a mid-size case, an 8-layer stack with
a heavy-tailed length mix, a long-sequence training case and a ranking case
with appended candidates ("Model Architecture": the candidate is appended to
the history and compared with it in the same pass).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed: int
    B: int                      # sequences in the batch
    lengths: Tuple              # ("uniform", lo, hi) | ("zipf", a, lo, hi) | ("fixed", n_hist)
    D: int                      # model width
    H: int                      # heads
    d_qk: int
    d_v: int
    n_layers: int
    dtype: str                  # "f32" | "bf16"
    backward: bool              # fwd+bwd training step
    num_candidates: int = 0     # candidates appended to every sequence (0 = causal only)
    norm_len: int = 0           # length normaliser N (the config's maximum length)
    n_pos_buckets: int = 128
    n_time_buckets: int = 128
    gap_mean_s: float = 60.0    # mean of the exponential inter-event gaps, seconds
    t0_range: Tuple[int, int] = (1_600_000_000, 1_700_000_000)
    x_std: Optional[float] = None      # None -> 1/sqrt(D)
    rab_std: float = 0.02

    @property
    def f1_width(self) -> int:
        """Columns of the U|V|Q|K projection: H*(2*d_v + 2*d_qk)."""
        return self.H * (2 * self.d_v + 2 * self.d_qk)

    def unit_scale(self) -> "Config":
        """Stress variant: X ~ N(0,1), rab ~ N(0,1), N = 1 (weights unchanged)."""
        return dataclasses.replace(self, name=self.name + "-unit", x_std=1.0,
                                   rab_std=1.0, norm_len=1)

    def shrunk(self, B: int, lengths: Tuple, num_candidates: Optional[int] = None,
               n_layers: Optional[int] = None, suffix: str = "-small") -> "Config":
        """Same widths, fewer/shorter sequences (for oracle-sized parity runs)."""
        return dataclasses.replace(
            self, name=self.name + suffix, B=B, lengths=lengths,
            num_candidates=self.num_candidates if num_candidates is None else num_candidates,
            n_layers=self.n_layers if n_layers is None else n_layers)


CONFIGS = {
    1: Config("c1-f32-1layer", seed=1, B=4, lengths=("uniform", 16, 128), D=64, H=2,
              d_qk=32, d_v=32, n_layers=1, dtype="f32", backward=False, norm_len=128),
    2: Config("c2-bf16-1layer", seed=2, B=32, lengths=("uniform", 64, 1024), D=256, H=4,
              d_qk=64, d_v=64, n_layers=1, dtype="bf16", backward=False, norm_len=1024),
    3: Config("c3-bf16-8layer-zipf", seed=3, B=64, lengths=("zipf", 1.2, 32, 2048), D=512,
              H=8, d_qk=64, d_v=64, n_layers=8, dtype="bf16", backward=False, norm_len=2048),
    4: Config("c4-bf16-train", seed=4, B=8, lengths=("uniform", 4096, 8192), D=512, H=4,
              d_qk=128, d_v=128, n_layers=1, dtype="bf16", backward=True, norm_len=8192),
    5: Config("c5-bf16-ranking", seed=5, B=16, lengths=("fixed", 4096), D=256, H=4,
              d_qk=64, d_v=64, n_layers=4, dtype="bf16", backward=False,
              num_candidates=512, norm_len=4608),
}


def get_config(i: int) -> Config:
    return CONFIGS[i]
