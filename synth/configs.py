"""The five workload configurations of the quantizer (DiT linear-layer inputs).

Shapes follow the widths of the three DiTs the KroQuant abstract evaluates
(PixArt-Sigma 1152, SANA-1600M 2240, FLUX.1-schnell 3072 / 12288); the value
model (per-token mean from adaLN-style conditioning plus a few outlier channels)
stands in for real activations, which need trained checkpoints and prompt sets.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    name: str
    rows: int
    d: int
    dtype: str              # "bf16" or "fp32"
    dist: str               # "gauss_mean" or "student_t"
    mean_std: float         # std of the per-token mean m_t (gauss_mean only)
    outlier_frac: float
    outlier_scale: float
    seed: int
    t_nu: float = 3.0
    sq: bool = False        # also exercise the SmoothQuant baseline
    identity: bool = False  # also exercise all-identity factors
    extra: dict = field(default_factory=dict)

    @property
    def nb(self) -> int:
        return self.d // 32

    @property
    def elements(self) -> int:
        return self.rows * self.d

    @property
    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.d))


CONFIGS = {
    # tiny fp32 case the oracle finishes instantly
    "tiny": Config("tiny", 256, 1152, "fp32", "gauss_mean", 2.0, 0.01, 30.0, seed=0),
    # PixArt-Sigma 1024px: 128x128 latent, patch 2 -> 4096 tokens, width 1152
    "pixart": Config("pixart", 4096, 1152, "bf16", "gauss_mean", 2.0, 0.01, 30.0, seed=1,
                     sq=True, identity=True),
    # SANA-1600M-like: batch 2 x 1024 tokens, width 2240, heavy tails
    "sana": Config("sana", 2048, 2240, "bf16", "student_t", 0.0, 0.005, 50.0, seed=2),
    # FLUX.1-schnell-like joint stream: 4096 image + 512 text tokens, width 3072
    "flux": Config("flux", 4608, 3072, "bf16", "gauss_mean", 3.0, 0.01, 40.0, seed=3, sq=True),
    # FLUX MLP input: width 12288
    "flux_mlp": Config("flux_mlp", 4608, 12288, "bf16", "gauss_mean", 3.0, 0.01, 40.0, seed=3),
    # batch-4 FLUX shapes, one denoising step's worth of layer calls
    "flux_b4": Config("flux_b4", 4 * 4608, 3072, "bf16", "gauss_mean", 3.0, 0.01, 40.0, seed=4000),
    "flux_b4_mlp": Config("flux_b4_mlp", 4 * 4608, 12288, "bf16", "gauss_mean", 3.0, 0.01, 40.0,
                          seed=4001),
}

# The batched sweep: 28 calls alternating the two batch-4 shapes, each with its
# own inputs and factor set (seed 4000 + call index).
SWEEP_CALLS = 28


def sweep_call(i: int) -> Config:
    base = CONFIGS["flux_b4"] if i % 2 == 0 else CONFIGS["flux_b4_mlp"]
    return Config(f"sweep{i}", base.rows, base.d, base.dtype, base.dist, base.mean_std,
                  base.outlier_frac, base.outlier_scale, seed=4000 + i)


def get_config(name: str) -> Config:
    return CONFIGS[name]


@dataclass(frozen=True)
class WeightConfig:
    """A linear layer's weight W[rows = output channels][d = input channels]; the
    quantizer's blocks run along d, matching the activations that layer takes."""
    name: str
    rows: int
    d: int
    dtype: str
    std: float              # base standard deviation of the entries
    row_spread: float       # per-output-row std multiplier exp(N(0, row_spread))
    seed: int

    @property
    def nb(self) -> int:
        return self.d // 32


WEIGHT_CONFIGS = {
    # small fp32 case for the oracle
    "tiny_w": WeightConfig("tiny_w", 192, 1152, "fp32", 0.02, 0.3, seed=20),
    # PixArt-Sigma attention projection 1152 -> 1152
    "pixart_w": WeightConfig("pixart_w", 1152, 1152, "bf16", 0.02, 0.3, seed=21),
    # FLUX.1-schnell joint-stream MLP up-projection 3072 -> 12288 (input width 3072)
    "flux_w_mlp": WeightConfig("flux_w_mlp", 12288, 3072, "bf16", 0.02, 0.3, seed=22),
    # FLUX.1-schnell MLP down-projection 12288 -> 3072 (input width 12288)
    "flux_w_down": WeightConfig("flux_w_down", 3072, 12288, "bf16", 0.01, 0.3, seed=23),
}


def get_weight_config(name: str) -> WeightConfig:
    return WEIGHT_CONFIGS[name]
