"""The five workload shapes and their value distributions.

c0  tiny fp32:        batch 1,   D 16,   N 4,  L 64      (plus the 2-state impulse case)
c1  130M-shaped fp32: batch 8,   D 1536, N 16, L 2048    gate on
c2  long bf16:        batch 1,   D 2048, N 16, L 65536   gate on, no D-skip
c3  2.8B-shaped bf16: batch 16,  D 5120, N 16, L 2048    A jitter N(0, 0.1^2), gate on
c4  decode bf16:      batch 256, D 5120, N 16, 64 one-token steps, fp32 state
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    dim: int
    dstate: int
    seqlen: int
    dtype: str            # "f32" or "bf16": storage of u, delta, B, C, z, y
    seed: int
    delta_std: float = 0.5
    a_jitter: float = 0.0
    gate: bool = True
    dskip: bool = True

    @property
    def elements(self) -> int:
        return self.batch * self.dim * self.seqlen


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    dim: int
    dstate: int
    steps: int
    dtype: str
    seed: int
    h0_std: float = 0.1
    delta_std: float = 1.0
    gate: bool = True
    dskip: bool = True


SCAN_CONFIGS = {
    "c0": ScanConfig("c0", 1, 16, 4, 64, "f32", seed=0, gate=False, dskip=True),
    "c1": ScanConfig("c1", 8, 1536, 16, 2048, "f32", seed=1),
    "c2": ScanConfig("c2", 1, 2048, 16, 65536, "bf16", seed=2, dskip=False),
    "c3": ScanConfig("c3", 16, 5120, 16, 2048, "bf16", seed=3, a_jitter=0.1),
}
DECODE_CONFIG = DecodeConfig("c4", 256, 5120, 16, 64, "bf16", seed=4)


@dataclass(frozen=True)
class SsdConfig:
    """A scalar-A-per-head (SSD) workload: nheads heads of headdim channels."""
    name: str
    batch: int
    nheads: int
    headdim: int
    dstate: int
    seqlen: int
    dtype: str
    seed: int
    delta_std: float = 0.5
    gate: bool = True
    dskip: bool = True

    @property
    def dim(self) -> int:
        return self.nheads * self.headdim

    @property
    def elements(self) -> int:
        return self.batch * self.dim * self.seqlen


# the 2.8B-shaped token grid of c3 (batch 16, D 5120, L 2048) as 80 heads of 64
# channels with 128 states
SSD_CONFIG = SsdConfig("c5", 16, 80, 64, 128, 2048, "bf16", seed=5)
CONFIGS = dict(SCAN_CONFIGS, c4=DECODE_CONFIG)


def get_config(name: str):
    return CONFIGS[name]
