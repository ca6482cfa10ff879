"""Pins of the oracle's expert FFN and combine (no GPU).

* a hand-worked two-expert example (tests/golden/ffn_hand_worked.json) that
  fixes the gate|up split, the operand orientation of w1 / w2 and the k order
  of the weights;
* with one expert and K = 1 the layer is the dense SwiGLU MLP, computed with
  torch.nn.functional (a library composition independent of the oracle);
* with identity experts (y = x) combine returns sum_k w_k x_t, and with K = 1,
  w = 1 dispatch -> combine is a pure permutation round trip;
* silu special values.
"""
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from synth import MoEConfig, MoEInputs, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs_from_lists(g, H, I, E, K, tile=1):
    cfg = MoEConfig("hand", len(g["x"]), H, I, E, 0, E, K, tile)
    return MoEInputs(
        cfg, 0,
        torch.tensor(g["x"], dtype=torch.float32).to(torch.bfloat16),
        torch.tensor(g["topk_idx"], dtype=torch.int32),
        torch.tensor(g["topk_weights"], dtype=torch.float32),
        torch.tensor(g["w1"], dtype=torch.float32).to(torch.bfloat16), None,
        torch.tensor(g["w2"], dtype=torch.float32).to(torch.bfloat16), None,
    )


def test_hand_worked_two_experts():
    g = json.load(open(os.path.join(GOLDEN, "ffn_hand_worked.json")))
    inp = _inputs_from_lists(g, H=2, I=1, E=2, K=2)
    res = oracle.moe_layer(inp)
    np.testing.assert_allclose(res.out, np.array(g["out"]), rtol=1e-13, atol=1e-13)
    # the intermediate h of each pair
    x = oracle.bf16_to_f64(inp.x)
    pairs = [(0, 0), (0, 1), (1, 1), (1, 0)]
    for (t, e), h_ref in zip(pairs, g["h"]):
        W1 = oracle.bf16_to_f64(inp.w1[e])
        G = x[t] @ W1.T
        assert math.isclose(oracle.silu(G[:1])[0] * G[1], h_ref, rel_tol=1e-13)


def test_single_expert_is_dense_swiglu_mlp():
    cfg = MoEConfig("dense", 37, 96, 48, 1, 0, 1, 1, 16)
    inp = make_inputs(cfg, 21)
    inp.topk_weights = torch.ones_like(inp.topk_weights)
    res = oracle.moe_layer(inp)
    x = inp.x.to(torch.float64)
    w1 = inp.w1[0].to(torch.float64)
    w2 = inp.w2[0].to(torch.float64)
    gate = F.linear(x, w1[:48])
    up = F.linear(x, w1[48:])
    ref = F.linear(F.silu(gate) * up, w2)
    np.testing.assert_allclose(res.out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_sampled_tokens_match_full_layer():
    cfg = MoEConfig("sample", 50, 64, 32, 6, 1, 4, 3, 8)   # experts 1..4 local of 0..5
    inp = make_inputs(cfg, 4)
    full = oracle.moe_layer(inp)
    toks = [0, 7, 13, 49]
    part = oracle.moe_layer(inp, tokens=toks)
    np.testing.assert_allclose(part.out, full.out[toks], rtol=1e-12, atol=1e-14)  # BLAS blocking may differ


def test_identity_experts_combine_is_weighted_sum_of_x():
    cfg = MoEConfig("ident", 40, 24, 8, 7, 2, 3, 4, 4)     # experts 2..4 local
    inp = make_inputs(cfg, 9, weights=False)
    p = oracle.plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    rows, payload = oracle.dispatch(inp.x, p, fp8=False)
    pool = np.zeros((p.P_cap, cfg.H), dtype=np.float64)
    pool[rows] = (payload.astype(np.uint32) << 16).view(np.float32)
    # identity expert: y_pool = pool; gather each pair's row back
    pos = p.pos.reshape(cfg.T, cfg.K)
    local = pos >= 0
    y_pair = np.where(local[:, :, None], pool[np.maximum(pos, 0)], 0.0)
    out = oracle.combine(y_pair, inp.topk_weights, local)
    w = inp.topk_weights.numpy().astype(np.float64)
    x = oracle.bf16_to_f64(inp.x)
    ref = (w * local).sum(axis=1)[:, None] * x
    np.testing.assert_allclose(out, ref, rtol=1e-15, atol=0)
    assert (out[~local.any(axis=1)] == 0).all()


def test_permutation_round_trip_k1():
    cfg = MoEConfig("perm", 33, 16, 8, 5, 0, 5, 1, 4)
    inp = make_inputs(cfg, 2, weights=False)
    p = oracle.plan(inp.topk_idx, 0, 5, 4)
    rows, payload = oracle.dispatch(inp.x, p, fp8=False)
    back = np.zeros((cfg.T, cfg.H), dtype=np.uint16)
    back[p.src[rows] // cfg.K] = payload
    assert np.array_equal(back, oracle.bf16_bits(inp.x))


def test_silu_special_values():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 800.0, -800.0])
    s = oracle.silu(z)
    assert s[0] == 0.0
    assert math.isclose(s[1], 1 / (1 + math.exp(-1)), rel_tol=1e-15)
    assert math.isclose(s[1] - s[2], 1.0, rel_tol=1e-15)      # silu(z) - silu(-z) = z
    assert math.isclose(s[3], 40.0, rel_tol=1e-15)
    assert abs(s[4]) < 1e-15
    assert s[5] == 800.0 and s[6] == 0.0


def test_fp8_layer_with_exact_values_equals_bf16_layer_up_to_h_rounding():
    # x holds e4m3-exact values with 448 in every group (scale 1); weights are e4m3
    # values with block scale 1, so GEMM A sees the same operands on both paths and
    # only h's quantisation differs (bounded by half a 3-bit mantissa step).
    cfg8 = MoEConfig("exact8", 6, 128, 128, 2, 0, 2, 1, 4, "fp8")
    rng = np.random.default_rng(1)
    codes = rng.integers(0x20, 0x50, size=(6, 128)).astype(np.uint8)
    codes[:, 0] = 0x7E
    x = torch.from_numpy(oracle.e4m3_decode(codes).astype(np.float32)).to(torch.bfloat16)
    w1c = torch.from_numpy(rng.integers(0x18, 0x30, size=(2, 256, 128)).astype(np.uint8))
    w2c = torch.from_numpy(rng.integers(0x18, 0x30, size=(2, 128, 128)).astype(np.uint8))
    ones1 = torch.ones(2, 2, 1)
    ones2 = torch.ones(2, 1, 1)
    idx = torch.tensor([[0], [1], [0], [1], [1], [0]], dtype=torch.int32)
    w = torch.ones(6, 1)
    inp8 = MoEInputs(cfg8, 0, x, idx, w, w1c.view(torch.float8_e4m3fn), ones1,
                     w2c.view(torch.float8_e4m3fn), ones2)
    cfgb = cfg8.with_(dtype="bf16")
    w1b = torch.from_numpy(oracle.e4m3_decode(w1c.numpy()).astype(np.float32)).to(torch.bfloat16)
    w2b = torch.from_numpy(oracle.e4m3_decode(w2c.numpy()).astype(np.float32)).to(torch.bfloat16)
    inpb = MoEInputs(cfgb, 0, x, idx, w, w1b, None, w2b, None)
    o8 = oracle.moe_layer(inp8).out
    ob = oracle.moe_layer(inpb).out
    err = oracle.max_norm_rel_err(o8, ob)
    assert 0 < err < 2.0 ** -4
