"""Seeded synthetic inputs for the KroQuant quantizer (shared by tests, bench, smoke).

This package draws activations, weights, factor parameters and SmoothQuant
multipliers.
It holds none of the quantizer's arithmetic and imports neither the oracle nor
the GPU library.
"""
from .configs import (  # noqa: F401
    CONFIGS, WEIGHT_CONFIGS, Config, WeightConfig, get_config, get_weight_config,
)
from .gen import (  # noqa: F401
    bf16_bits_from_f32, f32_from_bf16_bits, make_activations, make_activations_device, make_params,
    make_identity_params, make_rotation_params,
    make_sq_mult, make_inputs, make_weights, make_modulation,
)
