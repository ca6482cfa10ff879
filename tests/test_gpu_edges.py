"""Degenerate layers on the GPU against the oracle (bf16 1e-2, fp8 / mxfp4 3e-2, plan
bit-exact): no local pair at all (the FFN sees zero tiles; out is exactly zero, and so
are all gradients of the training path), a single token, the largest local expert
count (1024), and one expert taking every pair."""
import dataclasses

import numpy as np
import pytest
import torch

import combine_moe_dispatch_02_amd as moe
import oracle
from synth import MoEConfig, make_dout, make_inputs

from _gpu import TOL, assert_plan_equal, dev_inputs, make_layer, out_rows_f64, rel_err, run_layer, say

pytestmark = pytest.mark.gpu


def _routed(inp, idx):
    """The same inputs with another routing (weights and x unchanged)."""
    return dataclasses.replace(inp, topk_idx=idx.to(torch.int32).contiguous())


NO_LOCAL = [
    MoEConfig("no_local_bf16", 50, 256, 128, 16, 0, 8, 4, 16),
    MoEConfig("no_local_fp8", 50, 512, 256, 16, 0, 8, 4, 64, "fp8"),
    MoEConfig("no_local_mx", 50, 512, 256, 16, 0, 8, 4, 128, "mxfp4"),
]


@pytest.mark.parametrize("cfg", NO_LOCAL, ids=[c.name for c in NO_LOCAL])
def test_layer_without_local_pairs(cfg):
    inp = make_inputs(cfg)
    # every pair goes to experts 8..11, none of which is local
    inp = _routed(inp, 8 + torch.arange(cfg.K).repeat(cfg.T, 1))
    d = dev_inputs(inp)
    layer = make_layer(cfg)
    say("layer without local pairs", cfg.name)
    out = run_layer(layer, d)
    op = oracle.plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    assert op.P == 0
    assert_plan_equal(layer.plan, op)
    assert not bool(out.float().abs().sum())


def test_training_without_local_pairs():
    cfg = NO_LOCAL[0].with_(name="no_local_train", tile=64, H=512, I=512)
    inp = _routed(make_inputs(cfg), 8 + torch.arange(cfg.K).repeat(cfg.T, 1))
    d = dev_inputs(inp)
    layer = make_layer(cfg, train=True)
    w1, w2, _, _ = layer.prepare_weights(d["w1"], d["w2"])
    w1t, w2t = layer.prepare_backward_weights(d["w1"], d["w2"])
    say("training without local pairs")
    out = layer.forward(d["x"], d["idx"], d["w"], w1, w2)
    dx, dw, dW1, dW2 = layer.backward(make_dout(cfg, inp.seed).cuda(), d["w"], w1t, w2t)
    torch.cuda.synchronize()
    assert moe.moe_get_error(layer.ws) == 0
    for name, t in (("out", out), ("dx", dx), ("dw", dw), ("dW1", dW1), ("dW2", dW2)):
        assert not bool(t.float().abs().sum()), name


ONE_TOKEN = [
    MoEConfig("one_token_k1", 1, 256, 128, 8, 0, 8, 1, 16),
    MoEConfig("one_token_k8", 1, 1024, 512, 8, 0, 8, 8, 128),            # big-tile kernels, 8 one-row tiles
    MoEConfig("one_token_fp8", 1, 512, 256, 8, 0, 8, 4, 64, "fp8"),
    MoEConfig("one_token_mx", 1, 512, 256, 8, 0, 8, 4, 128, "mxfp4"),
]

EXTREME = [
    MoEConfig("e1024", 300, 128, 64, 1024, 0, 1024, 4, 16),              # the largest local expert count
    MoEConfig("e1024_ep", 300, 128, 64, 2048, 1024, 1024, 8, 16),         # ids 1024..2047 local
]


@pytest.mark.parametrize("cfg", ONE_TOKEN + EXTREME, ids=[c.name for c in ONE_TOKEN + EXTREME])
def test_layer_degenerate_shapes(cfg):
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    layer = make_layer(cfg)
    say("degenerate layer", cfg.name)
    out = run_layer(layer, d)
    ref = oracle.moe_layer(inp)
    assert_plan_equal(layer.plan, ref.plan)
    none_local = ~(ref.plan.pos.reshape(cfg.T, cfg.K) >= 0).any(axis=1)
    got = out_rows_f64(out)
    assert (got[none_local] == 0).all()
    if np.abs(ref.out).max() > 0:
        err = rel_err(got, ref.out)
        print(f"{cfg.name}: max-norm rel err {err:.3e}")
        assert err <= TOL[cfg.dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "mxfp4"])
def test_layer_one_expert_takes_every_pair(dtype):
    # K = 1 and every token on local expert 3: one segment of ceil(1000/128) = 8 tiles, the
    # last one ragged, and seven experts with no rows
    cfg = MoEConfig(f"one_expert_{dtype}", 1000, 512, 256, 8, 0, 8, 1, 128, dtype)
    inp = _routed(make_inputs(cfg), torch.full((cfg.T, 1), 3))
    d = dev_inputs(inp)
    layer = make_layer(cfg)
    say("layer with one expert taking every pair", dtype)
    out = run_layer(layer, d)
    ref = oracle.moe_layer(inp)
    assert_plan_equal(layer.plan, ref.plan)
    assert ref.plan.P == 1024
    err = rel_err(out_rows_f64(out), ref.out)
    print(f"{cfg.name}: max-norm rel err {err:.3e}")
    assert err <= TOL[dtype]


POISON = [
    MoEConfig("poison_bf16", 700, 1024, 512, 9, 1, 6, 4, 128),            # big-tile kernels, EP slice
    MoEConfig("poison_bf16_t32", 333, 384, 192, 9, 0, 9, 3, 32),          # general kernel
    MoEConfig("poison_fp8", 700, 1024, 512, 10, 1, 8, 4, 128, "fp8"),
    MoEConfig("poison_mx", 700, 1024, 768, 10, 1, 8, 4, 128, "mxfp4"),
]


def poison_(t):
    """Fill with all-ones bytes: NaN as bf16, e4m3 and fp32."""
    t.view(torch.uint8).fill_(0xFF)


def poison_workspace_h(layer):
    """NaN bytes over h and its scales (the workspace past what plan and dispatch use)."""
    plan_end = moe.workspace_bytes(layer.T, layer.K, layer.E_local, layer.tile, layer.pool_rows, 0, layer.dtype)
    layer.ws.buf[plan_end:].fill_(0xFF)


@pytest.mark.parametrize("cfg", POISON, ids=[c.name for c in POISON])
def test_padding_rows_never_reach_the_output(cfg):
    # padding rows of the pool, of h and of y_pool hold NaN before the call: no output element
    # may see one (every GEMM output row depends only on its own input row, combine reads real
    # rows only)
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    layer = make_layer(cfg)
    for t in (layer.pool, layer.y_pool) + ((layer.pool_s,) if layer.pool_s is not None else ()):
        poison_(t)
    poison_workspace_h(layer)
    say("poisoned padding", cfg.name)
    out = run_layer(layer, d)
    ref = oracle.moe_layer(inp)
    assert_plan_equal(layer.plan, ref.plan)
    got = out_rows_f64(out)
    assert np.isfinite(got).all()
    assert (layer.plan.offsets[-1].item() % cfg.tile == 0)
    src = layer.plan.src.cpu().numpy()[: layer.plan.offsets[-1].item()]
    assert (src < 0).any(), "the case has padding rows"
    err = rel_err(got, ref.out)
    print(f"{cfg.name} (poisoned padding): max-norm rel err {err:.3e}")
    assert err <= TOL[cfg.dtype]
