"""The five synthetic workloads the library is measured and parity-tested on.

Shapes follow the video DiTs the TRA pages validate on (Wan2.1 1.3B/14B and
HunyuanVideo 13B latent grids, "Token Radius Attention for Efficient Video
Generation", section 3 contribution 4 and section 4); the activations are
synthetic (``synth.py``).  tau values for workloads 2-4 are calibrated to the
stated block density (retained token pairs / all token pairs) by
``tests/golden/calibrate_tau.py`` with the CPU oracle on a seeded sample of
q-blocks (``tests/golden/tau_calibration.json``), then frozen here; so are the
static-mask workload's entropy values, one per head, each bisected to the density
the same head of workload 3 reaches.
"""
from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    batch: int
    heads: int
    D: int
    dtype: str          # "f32" or "bf16"
    F: int
    H: int
    W: int
    block_q: int
    block_k: int
    tau: float
    gamma: float = 0.5
    vote_threshold: int = 1
    tile_h: int = 8
    tile_w: int = 8
    t_lo: float = 0.25
    t_hi: float = 8.0
    density_target: float | None = None
    static_mask: bool = False   # one entropy value per head instead of per-query entropies
    static_entropy: tuple = ()  # those values (nats), one per (batch, head)

    @property
    def outer(self) -> int:
        return self.batch * self.heads

    @property
    def N(self) -> int:
        return self.F * self.H * self.W

    @property
    def nqb(self) -> int:
        return -(-self.N // self.block_q)

    @property
    def nkb(self) -> int:
        return -(-self.N // self.block_k)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def dense_flops(self) -> float:
        return 4.0 * self.outer * float(self.N) ** 2 * self.D


# entropy constant c_h of each head of the static radial-style mask (workload 5), from the
# calibration
STATIC_ENTROPY_W5 = (
    11.05, 11.05, 11.09, 10.83, 10.91, 11.08, 11.03, 10.99, 11.01, 10.99,
    10.98, 10.92, 10.94, 10.83, 11.08, 11.05, 10.99, 10.88, 10.83, 10.98,
    10.99, 11.01, 11.08, 10.92, 11.05, 11.05, 11.05, 11.02, 10.91, 10.99,
    11.07, 10.98, 10.98, 11.01, 10.83, 10.84, 10.99, 10.92, 10.94, 11.07,
)

WORKLOADS = {
    1: Workload(1, "tiny-4x16x16", 1, 2, 64, "f32", 4, 16, 16, 64, 64, tau=1.0),
    2: Workload(2, "wan2.1-1.3b-480p-21x30x52", 1, 12, 128, "bf16", 21, 30, 52, 128, 64, tau=1.23e-3,
                density_target=0.15),
    3: Workload(3, "wan2.1-14b-720p-21x45x80", 1, 40, 128, "bf16", 21, 45, 80, 128, 64, tau=3.01e-2,
                density_target=0.15),
    4: Workload(4, "hunyuanvideo-13b-720p-33x45x80", 1, 24, 128, "bf16", 33, 45, 80, 128, 64, tau=4.41e-2,
                t_lo=0.1, t_hi=16.0, density_target=0.15),
    5: Workload(5, "static-radial-21x45x80", 1, 40, 128, "bf16", 21, 45, 80, 128, 64, tau=3.01e-2,
                density_target=0.15, static_mask=True, static_entropy=STATIC_ENTROPY_W5),
}


# the headline workload at the ends of the 9-19% retained range (same calibration)
DENSITY_TAU = {3: {0.09: 3.57e-3, 0.15: 3.01e-2, 0.19: 6.95e-2}}


def get(wid: int) -> Workload:
    return WORKLOADS[wid]
