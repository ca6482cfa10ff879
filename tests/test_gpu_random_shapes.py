"""Seeded random layer shapes on the GPU against the oracle, over the shapes each path
accepts: bf16 on every tile (16/32/64/128; H a multiple of 128, I of 64), fp8 (tile 64 or
128; H % 256, I % 128), mxfp4 (tile 128; H % 512, I % 256); top-k 1..16, EP slices with
pairs to other GPUs, uniform or Zipf routing; and larger bf16 shapes of the 256-row units
(several tiles per expert). Every output element is compared (max-norm
relative error 1e-2 bf16, 3e-2 fp8 / mxfp4), the plan bit for bit, and tokens without a
local pair must be exactly zero."""
import random

import numpy as np
import pytest

import oracle
from synth import MoEConfig, make_inputs

from _gpu import TOL, assert_plan_equal, dev_inputs, make_layer, out_rows_f64, rel_err, run_layer, say

pytestmark = pytest.mark.gpu


def _shapes(n=18, seed=20261203):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        dtype = ("bf16", "bf16", "fp8", "mxfp4")[i % 4]
        if dtype == "bf16":
            tile = rng.choice([16, 32, 64, 128])
            H = 128 * rng.randint(1, 8)
            I = 64 * rng.randint(1, 8)
        elif dtype == "fp8":
            tile = rng.choice([64, 128])
            H = 256 * rng.randint(1, 4)
            I = 128 * rng.randint(1, 4)
        else:
            tile = 128
            H = 512 * rng.randint(1, 2)
            I = 256 * rng.randint(1, 2)
        E_local = rng.randint(1, 24)
        expert_begin = rng.choice([0, 0, rng.randint(1, 8)])
        num_experts = expert_begin + E_local + rng.choice([0, 0, rng.randint(1, 16)])
        K = rng.randint(1, min(16, num_experts))
        T = rng.randint(1, 400)
        routing = rng.choice(["uniform", "uniform", "zipf1.2"])
        out.append(MoEConfig(f"rand{i}_{dtype}_t{tile}", T, H, I, num_experts, expert_begin, E_local, K, tile,
                             dtype, routing))
    return out


def _sq_shapes(n=6, seed=78):
    """Seeded shapes of the 256-row units (bf16, tile 128, H % 256, I % 128): several tiles per
    expert, odd tile counts (one-tile units), EP slices, empty experts under Zipf routing, and
    I % 256 both zero (GEMM A launched on both unit shapes, the plan choosing) and not."""
    rng = random.Random(seed)
    out = []
    for i in range(n):
        H = 256 * rng.randint(1, 4)
        I = 128 * rng.randint(1, 4)
        E_local = rng.randint(2, 12)
        expert_begin = rng.choice([0, rng.randint(1, 6)])
        num_experts = expert_begin + E_local + rng.choice([0, rng.randint(1, 8)])
        K = rng.randint(1, min(8, num_experts))
        T = rng.randint(300, 1500)
        routing = rng.choice(["uniform", "zipf1.2"])
        out.append(MoEConfig(f"sqrand{i}_h{H}_i{I}", T, H, I, num_experts, expert_begin, E_local, K, 128,
                             "bf16", routing))
    return out


SHAPES = _shapes() + _sq_shapes()


@pytest.mark.parametrize("cfg", SHAPES, ids=[c.name for c in SHAPES])
def test_random_layer_shape(cfg):
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    layer = make_layer(cfg)
    say("random layer", cfg)
    out = run_layer(layer, d)
    ref = oracle.moe_layer(inp)
    assert_plan_equal(layer.plan, ref.plan)
    got = out_rows_f64(out)
    none_local = ~(ref.plan.pos.reshape(cfg.T, cfg.K) >= 0).any(axis=1)
    assert (got[none_local] == 0).all()
    if np.abs(ref.out).max() > 0:
        err = rel_err(got, ref.out)
        print(f"{cfg.name}: T {cfg.T} H {cfg.H} I {cfg.I} E {cfg.num_local_experts} K {cfg.K}: {err:.3e}")
        assert err <= TOL[cfg.dtype]
