"""The allocation-free plan entry point (moe_plan_noalloc, scratch in the library's static
device array) against moe_plan with a workspace, through the C ABI: every plan array bit
for bit, on two calls in a row, the second with a smaller input (the shared scratch keeps
the first call's contents), and against the oracle's plan."""
import numpy as np
import pytest
import torch

import combine_moe_dispatch_02_amd as moe
import oracle
from synth import MoEConfig, config_by_name, make_inputs

from _gpu import assert_plan_equal, say

pytestmark = pytest.mark.gpu

FIELDS = ("counts", "offsets", "pos", "src", "tile_expert", "num_tiles", "tile_ready")


def _plans(cfg):
    inp = make_inputs(cfg, weights=False)
    idx = inp.topk_idx.cuda()
    ref = moe.Plan.allocate(cfg.T, cfg.K, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    ws = moe.Workspace(cfg.T, cfg.K, cfg.num_local_experts, cfg.tile)
    moe.moe_plan(idx, ref, ws)
    got = moe.Plan.allocate(cfg.T, cfg.K, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    for t in (got.counts, got.offsets, got.pos, got.src, got.tile_expert, got.num_tiles, got.tile_ready):
        t.fill_(-7)                                   # every array must be written
    moe.moe_plan_noalloc(idx, got)
    torch.cuda.synchronize()
    return inp, ref, got


@pytest.mark.parametrize("first,second", [
    (config_by_name("zipf_skew"), config_by_name("decode")),                 # several plan blocks, then one
    (MoEConfig("na_ep", 8192, 64, 64, 256, 0, 32, 8, 128), config_by_name("tiny")),
])
def test_plan_noalloc_matches_plan(first, second):
    for cfg in (first, second):
        say("plan noalloc", cfg.name)
        inp, ref, got = _plans(cfg)
        for f in FIELDS:
            assert torch.equal(getattr(ref, f), getattr(got, f)), (cfg.name, f)
        assert_plan_equal(got, oracle.plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile))
