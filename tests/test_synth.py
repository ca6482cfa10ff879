"""The seeded generator: deterministic, with the stated shapes and distributions (no GPU)."""
import numpy as np
import torch

from synth import CONFIGS, config_by_name, expert_weights, make_inputs, make_routing, make_x
from synth.inputs import base_seed


def test_deterministic_and_seed_sensitive():
    cfg = config_by_name("tiny")
    a = make_inputs(cfg)
    b = make_inputs(cfg)
    c = make_inputs(cfg, seed=5)
    assert torch.equal(a.x, b.x) and torch.equal(a.w1, b.w1) and torch.equal(a.topk_idx, b.topk_idx)
    assert not torch.equal(a.x, c.x)
    assert a.seed == 1000 and base_seed(config_by_name("fp8_weights")) == 1004


def test_routing_distinct_and_softmax():
    for cfg in CONFIGS:
        idx, w = make_routing(cfg, base_seed(cfg))
        assert idx.shape == (cfg.T, cfg.K) and idx.dtype == torch.int32
        s = np.sort(idx.numpy(), axis=1)
        assert (np.diff(s, axis=1) > 0).all()
        assert idx.min() >= 0 and idx.max() < cfg.num_experts
        assert np.allclose(w.numpy().sum(axis=1), 1.0, atol=2e-7)
        assert (np.diff(w.numpy(), axis=1) <= 0).all()      # k = 0 is the largest


def test_zipf_workload_shape():
    cfg = config_by_name("zipf_skew")
    idx, _ = make_routing(cfg, base_seed(cfg))
    counts = np.bincount(idx.numpy().reshape(-1), minlength=cfg.num_experts)
    mean = cfg.T * cfg.K / cfg.num_experts
    assert counts.max() / mean > 8          # heavy head
    assert counts.min() <= 2                # near-empty tail
    assert counts.argmax() == 0


def test_ep_share_local_fraction():
    cfg = config_by_name("ep_share")
    idx, _ = make_routing(cfg, base_seed(cfg))
    frac = (idx.numpy() < 32).mean()
    assert 0.11 < frac < 0.14               # about 32/256 of the pairs


def test_weight_scale_and_subset_draw():
    cfg = config_by_name("tiny")
    inp = make_inputs(cfg)
    w1, _, w2, _ = expert_weights(cfg, inp.seed, 3)
    assert torch.equal(w1, inp.w1[3]) and torch.equal(w2, inp.w2[3])
    std1 = inp.w1.float().std().item()
    assert abs(std1 * np.sqrt(cfg.H) - 1) < 0.05
    x = make_x(cfg, inp.seed).float()
    assert abs(x.std().item() - 1) < 0.05


def test_fp8_weights_layout():
    cfg = config_by_name("fp8_weights").with_(name="fp8_small", T=16, H=256, I=128, num_experts=4,
                                               num_local_experts=4)
    inp = make_inputs(cfg, 3)
    assert inp.w1.dtype == torch.float8_e4m3fn and inp.w1.shape == (4, 256, 256)
    assert inp.w1_scale.shape == (4, 2, 2) and inp.w2_scale.shape == (4, 2, 1)
    # every block reaches +-448 in code space
    c = inp.w1.view(torch.uint8).reshape(4, 2, 128, 2, 128)
    assert ((c & 0x7F).amax(dim=(2, 4)) == 0x7E).all()


def test_mxfp4_weights_layout_and_rounding():
    # the stored weights are the MX quantisation of the fp32 masters: every block's
    # largest code is 6 or (rounded down from) 4..6, and each weight is within the
    # E2M1 rounding bound of its master (half the step at its magnitude, or the
    # saturation gap 6..8 for the block maximum)
    from oracle import dequantize_mx_fp4, unpack_fp4
    from synth.inputs import _mx_quant_e2m1

    cfg = config_by_name("mxfp4").with_(name="mx_small", T=16, H=256, I=128, num_experts=4,
                                         num_local_experts=4)
    inp = make_inputs(cfg, 3)
    assert inp.w1.dtype == torch.uint8 and inp.w1.shape == (4, 256, 128)
    assert inp.w1_scale.shape == (4, 256, 8) and inp.w2_scale.shape == (4, 256, 4)
    rng = np.random.default_rng(0)
    w = torch.from_numpy((rng.standard_normal((8, 128)) * 0.05).astype(np.float32))
    q, s = _mx_quant_e2m1(w)
    deq = dequantize_mx_fp4(q.numpy(), s.numpy())
    X = np.exp2(s.numpy().astype(np.float64) - 127).repeat(32, axis=1)
    a = np.abs(w.numpy().astype(np.float64)) / X
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    bound = np.where(a > 6, a - 6, step / 2) * X
    assert (np.abs(deq - w.numpy()) <= bound + 1e-30).all()
    codes = unpack_fp4(q.numpy()).reshape(8, 4, 32) & 7
    assert (codes.max(axis=2) >= 6).all()
