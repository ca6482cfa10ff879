"""A1 on the GPU: counts, offsets, pos, src, tile_expert and num_tiles are
bit-exact to the oracle's plan on every workload and on ragged / degenerate shapes."""
import numpy as np
import pytest
import torch

import combine_moe_dispatch_02_amd as moe
import oracle
from synth import CONFIGS, config_by_name, make_inputs

from _gpu import assert_plan_equal, say

pytestmark = pytest.mark.gpu


def gpu_plan(idx, expert_begin, E, tile, ws=None, plan=None):
    T, K = idx.shape
    plan = plan or moe.Plan.allocate(T, K, expert_begin, E, tile)
    ws = ws or moe.Workspace(T, K, E, tile)
    moe.moe_plan(idx.cuda(), plan, ws)
    torch.cuda.synchronize()
    return plan, ws


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c.name for c in CONFIGS])
def test_plan_workloads(cfg):
    inp = make_inputs(cfg, weights=False)
    say("plan", cfg.name)
    plan, _ = gpu_plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    op = oracle.plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    assert_plan_equal(plan, op)
    assert moe.moe_query_pool_rows(plan) == op.P


SHAPES = [
    # T, K, E_gen, expert_begin, E_local, tile
    (1, 1, 1, 0, 1, 16),
    (7, 3, 9, 2, 5, 32),
    (300, 8, 64, 0, 64, 64),
    (1000, 16, 40, 8, 17, 128),
    (5000, 4, 300, 100, 150, 16),
    (4097, 2, 1100, 0, 1024, 64),       # 1024 local experts, ragged pair count
    (777, 8, 3, 0, 3, 128),             # few experts, long segments
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_plan_random_shapes(shape):
    T, K, E_gen, eb, E, tile = shape
    g = torch.Generator().manual_seed(T * 31 + K)
    idx = torch.randint(-1, E_gen, (T, K), generator=g, dtype=torch.int32)
    say("plan shape", shape)
    plan, _ = gpu_plan(idx, eb, E, tile)
    assert_plan_equal(plan, oracle.plan(idx, eb, E, tile))


def test_plan_no_local_pairs():
    idx = torch.full((50, 4), 77, dtype=torch.int32)
    say("plan no local pairs")
    plan, _ = gpu_plan(idx, 0, 8, 16)
    op = oracle.plan(idx, 0, 8, 16)
    assert op.P == 0
    assert_plan_equal(plan, op)


def test_plan_all_to_one_expert():
    idx = torch.full((3000, 8), 5, dtype=torch.int32)
    idx[:, 1:] = -1
    say("plan all to one expert")
    plan, _ = gpu_plan(idx, 0, 8, 128)
    assert_plan_equal(plan, oracle.plan(idx, 0, 8, 128))


def test_plan_reuses_workspace():
    # the last-block counter resets itself: a second plan on the same buffers agrees
    cfg = config_by_name("zipf_skew")
    inp = make_inputs(cfg, weights=False)
    say("plan twice on one workspace")
    plan, ws = gpu_plan(inp.topk_idx, 0, cfg.num_local_experts, cfg.tile)
    idx2 = inp.topk_idx.flip(0).contiguous()
    plan, ws = gpu_plan(idx2, 0, cfg.num_local_experts, cfg.tile, ws=ws, plan=plan)
    assert_plan_equal(plan, oracle.plan(idx2, 0, cfg.num_local_experts, cfg.tile))
