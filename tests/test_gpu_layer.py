"""The whole path on the GPU (plan -> dispatch -> expert FFN -> combine) against the
oracle: max-normwise relative error <= 1e-2 (bf16) / 3e-2 (fp8, mxfp4), plan bit-exact,
tokens with no local pair exactly zero, repeated runs bitwise identical.

Small shapes are compared on every output element; the full-size workloads on a
seeded sample of tokens that the oracle computes one by one."""
import numpy as np
import pytest
import torch

import oracle
from synth import MoEConfig, config_by_name, make_inputs

from _gpu import (TOL, assert_plan_equal, dev_inputs, make_layer, out_rows_f64, rel_err, run_layer, say,
                  tile_covering_tokens)

pytestmark = pytest.mark.gpu

FULL_COMPARE = [
    config_by_name("tiny"),
    config_by_name("decode"),
    MoEConfig("ragged_t32", 333, 384, 192, 9, 0, 9, 3, 32),
    MoEConfig("ragged_t64", 517, 512, 320, 7, 2, 4, 2, 64),         # experts 2..5 local
    MoEConfig("t128_bn128", 1500, 640, 192, 5, 0, 5, 2, 128),       # H % 256 != 0, I % 128 != 0
    MoEConfig("t16_k16", 64, 256, 128, 20, 0, 20, 16, 16),
    MoEConfig("mix_bigY", 900, 1024, 384, 6, 0, 6, 2, 128),        # GEMM A general, GEMM Y big-tile
    MoEConfig("mix_bigA", 700, 640, 256, 5, 0, 5, 3, 64),          # GEMM A big-tile, GEMM Y general
    MoEConfig("big_both", 1200, 1024, 512, 9, 0, 9, 4, 128),
    MoEConfig("fp8_t64", 300, 512, 256, 6, 0, 6, 2, 64, "fp8"),
    MoEConfig("fp8_t128", 700, 1024, 384, 10, 1, 8, 4, 128, "fp8"),
    MoEConfig("fp8_big", 600, 1024, 512, 6, 0, 6, 2, 128, "fp8"),     # fp8 big-tile kernel, tiled weights
    MoEConfig("mx_small", 300, 512, 256, 4, 0, 4, 2, 128, "mxfp4"),   # mxfp4: one N block, 2 K steps
    MoEConfig("mx_big", 700, 1024, 768, 10, 1, 8, 4, 128, "mxfp4"),   # 3 A units, ragged tiles, EP slice
]


@pytest.mark.parametrize("cfg", FULL_COMPARE, ids=[c.name for c in FULL_COMPARE])
def test_layer_full_compare(cfg):
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    layer = make_layer(cfg)
    say("layer", cfg.name)
    out = run_layer(layer, d)
    ref = oracle.moe_layer(inp)
    assert_plan_equal(layer.plan, ref.plan)
    got = out_rows_f64(out)
    err = rel_err(got, ref.out)
    print(f"{cfg.name}: max-norm rel err {err:.3e}")
    assert err <= TOL[cfg.dtype]
    none_local = ~(ref.plan.pos.reshape(cfg.T, cfg.K) >= 0).any(axis=1)
    assert (got[none_local] == 0).all()


def _sample_tokens(cfg, inp, n=24, seed=0):
    rng = np.random.default_rng(seed)
    idx = inp.topk_idx.numpy()
    local = (idx >= cfg.expert_begin) & (idx < cfg.expert_begin + cfg.num_local_experts)
    pick = set(rng.choice(cfg.T, n, replace=False).tolist()) | {0, cfg.T - 1}
    pick.add(int(local.sum(axis=1).argmax()))
    if (~local.any(axis=1)).any():
        pick.add(int(np.nonzero(~local.any(axis=1))[0][0]))
    if cfg.routing == "zipf1.2":
        pick.add(int(np.nonzero((idx == 0).any(axis=1))[0][-1]))      # hottest expert's last tile
    return np.array(sorted(pick))


@pytest.mark.parametrize("name", ["ep_share", "zipf_skew", "fp8_weights", "mxfp4"])
def test_layer_full_size_sampled(name):
    # every pool tile has a compared pair (the token of its last real row), so a unit-mapping,
    # tail or scale-word error confined to some tiles cannot hide in an unsampled one
    cfg = config_by_name(name)
    inp = make_inputs(cfg, pin_memory=True)
    d = dev_inputs(inp)
    layer = make_layer(cfg)
    say("layer full size", name)
    out = run_layer(layer, d)
    p = oracle.plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    assert_plan_equal(layer.plan, p)
    toks = tile_covering_tokens(cfg, inp, p, _sample_tokens(cfg, inp))
    ref = oracle.moe_layer(inp, tokens=toks, p=p)
    got = out_rows_f64(out, toks)
    err = rel_err(got, ref.out)
    print(f"{name}: {len(toks)} tokens covering all {p.num_tiles} tiles, max-norm rel err {err:.3e}")
    assert err <= TOL[cfg.dtype]
    none_local = ~(p.pos.reshape(cfg.T, cfg.K) >= 0).any(axis=1)
    if none_local.any():
        zero_rows = torch.as_tensor(np.nonzero(none_local)[0], device="cuda")
        assert bool((out[zero_rows].float() == 0).all())


def test_layer_repeat_is_bitwise_identical():
    cfg = config_by_name("fp8_weights").with_(name="fp8_repeat", T=2048)
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    layer = make_layer(cfg)
    say("repeat determinism")
    a = run_layer(layer, d).clone()
    b = run_layer(layer, d).clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_layer_polled_pool_size_matches_bound():
    # the one host poll sizes the pool exactly; results match the sync-free bound
    cfg = config_by_name("ep_share").with_(name="ep_polled", T=1024)
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    big = make_layer(cfg)
    say("polled pool size")
    a = run_layer(big, d).clone()
    import combine_moe_dispatch_02_amd as moe
    P = moe.moe_query_pool_rows(big.plan)
    small = make_layer(cfg, pool_rows=P)
    b = run_layer(small, d)
    assert small.pool.shape[0] == P < big.pool.shape[0]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", ["decode", "big_both", "fp8_big"])
def test_layer_row_major_weights_on_big_tiles(name):
    # the big-tile kernel also reads row-major weights (fp8: row-major weights take the
    # general kernel); same tolerance as the tiled path
    cfg = config_by_name("decode") if name == "decode" else next(c for c in FULL_COMPARE if c.name == name)
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    layer = make_layer(cfg, weight_layout="row_major")
    assert not layer.tiled
    say("layer row-major weights", cfg.name)
    out = run_layer(layer, d)
    ref = oracle.moe_layer(inp)
    err = rel_err(out_rows_f64(out), ref.out)
    print(f"{cfg.name} row-major: max-norm rel err {err:.3e}")
    assert err <= TOL[cfg.dtype]


@pytest.mark.parametrize("order", [1, 2, 4, 7])
def test_layer_unit_walks_agree(order):
    # every walk of the (tile, N block) units computes the same bits as the default
    cfg = next(c for c in FULL_COMPARE if c.name == "big_both")
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    say("unit walk", order)
    ref = run_layer(make_layer(cfg), d).clone()
    import combine_moe_dispatch_02_amd as moe
    got = run_layer(make_layer(cfg, cfg=moe.TileConfig(0, 0, 0, order, 0)), d)
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))


@pytest.mark.parametrize("name", ["big_both", "mx_big"])
def test_layer_a_pipelines_agree(name):
    # the four-stage pool-row ring and the two-stage pipeline feed the MFMAs the same
    # operands in the same order: bitwise equal outputs
    import combine_moe_dispatch_02_amd as moe
    cfg = next(c for c in FULL_COMPARE if c.name == name)
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    say("A pipeline depth", name)
    ring = run_layer(make_layer(cfg, cfg=moe.TileConfig(0, 0, 0, 0, 0, 4)), d).clone()
    two = run_layer(make_layer(cfg, cfg=moe.TileConfig(0, 0, 0, 0, 0, 2)), d)
    assert torch.equal(ring.view(torch.int16), two.view(torch.int16))


def test_layer_large_batch_sampled():
    # four times the skew workload's pairs (524 288; a pool of about 540 k rows, 4.4 GB of bf16
    # pool rows and as much y): every 64-bit row offset and every per-tile buffer range at a
    # size past 2^32 bytes, on sampled tokens
    cfg = config_by_name("zipf_skew").with_(name="large_batch", T=65536, routing="uniform")
    inp = make_inputs(cfg, pin_memory=True)
    d = dev_inputs(inp)
    layer = make_layer(cfg)
    say("layer large batch", cfg.T)
    out = run_layer(layer, d)
    p = oracle.plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    assert_plan_equal(layer.plan, p)
    assert p.P * cfg.H * 2 > (1 << 32)
    toks = tile_covering_tokens(cfg, inp, p, _sample_tokens(cfg, inp, n=12))
    ref = oracle.moe_layer(inp, tokens=toks, p=p)
    err = rel_err(out_rows_f64(out, toks), ref.out)
    print(f"large batch: {len(toks)} tokens covering all {p.num_tiles} tiles, max-norm rel err {err:.3e}")
    assert err <= TOL[cfg.dtype]


SQ_CASES = [
    next(c for c in FULL_COMPARE if c.name == "big_both"),
    MoEConfig("sq_ep_odd", 1000, 1024, 384, 12, 3, 7, 3, 128),        # EP slice, odd tile counts
    MoEConfig("sq_zipf", 3000, 512, 256, 16, 0, 16, 4, 128, "bf16", "zipf1.2"),   # empty experts
]


@pytest.mark.parametrize("name", ["ep_share", "big_both"])
def test_layer_auto_unit_shape(name):
    # with the unit shape left to the library, GEMM A runs on whichever kernel the plan picks
    # on the device (ep_share: the 128-row units; big_both: the 256-row ones): the same bits as
    # either shape forced
    import combine_moe_dispatch_02_amd as moe
    cfg = config_by_name(name) if name == "ep_share" else next(c for c in FULL_COMPARE if c.name == name)
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    say("auto unit shape", cfg.name)
    auto = run_layer(make_layer(cfg), d).clone()
    for rows in (128, 256):
        got = run_layer(make_layer(cfg, cfg=moe.TileConfig(0, 0, 0, 0, 0, 0, 0, rows)), d)
        assert torch.equal(auto.view(torch.int16), got.view(torch.int16)), rows


@pytest.mark.parametrize("cfg", SQ_CASES, ids=[c.name for c in SQ_CASES])
def test_layer_unit_rows_agree(cfg):
    # the 256 x 256 units (two pool tiles, both operands by LDS-DMA) run the same MFMA chain
    # per output element as the 128 x 512 units: bitwise equal out, for every walk grouping;
    # and within tolerance of the oracle on every element
    import combine_moe_dispatch_02_amd as moe
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    say("unit rows", cfg.name)
    ref = run_layer(make_layer(cfg, cfg=moe.TileConfig(0, 0, 0, 0, 0, 0, 0, 128)), d).clone()
    for order in (0, 1, 3, 8):
        got = run_layer(make_layer(cfg, cfg=moe.TileConfig(0, 0, 0, order, 0, 0, 0, 256)), d)
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), order
    err = rel_err(out_rows_f64(got), oracle.moe_layer(inp).out)
    print(f"{cfg.name}: max-norm rel err {err:.3e}")
    assert err <= TOL[cfg.dtype]


MANY_UNITS = [
    MoEConfig("sq_many", 2000, 1024, 512, 8, 0, 8, 4, 128),            # 256-row units, ~140 per GEMM
    MoEConfig("fp8_many", 2000, 1024, 512, 8, 0, 8, 4, 128, "fp8"),    # big-tile kernel, ~250 GEMM A units
    MoEConfig("mx_many", 2000, 1024, 512, 8, 0, 8, 4, 128, "mxfp4"),
]


@pytest.mark.parametrize("cfg", MANY_UNITS, ids=[c.name for c in MANY_UNITS])
def test_layer_one_workgroup_walks_every_unit(cfg):
    # with a one-workgroup GEMM grid the workgroup walks more units than its table of units
    # decoded at start holds (64), so the later ones are found one by one: the same bits as
    # the full grid, and within tolerance of the oracle
    import combine_moe_dispatch_02_amd as moe
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    say("one-workgroup grid", cfg.name)
    ref = run_layer(make_layer(cfg), d).clone()
    got = run_layer(make_layer(cfg, cfg=moe.TileConfig(0, 1, 0, 0, 0)), d)
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
    want = oracle.moe_layer(inp)
    assert rel_err(out_rows_f64(got), want.out) <= TOL[cfg.dtype]
