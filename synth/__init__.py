"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the CPU oracle."""
from .inputs import (  # noqa: F401
    CONFIGS,
    MoEConfig,
    MoEInputs,
    config_by_name,
    expert_weights,
    make_dout,
    make_inputs,
    make_routing,
    make_x,
)
