"""Combine on completion (moe_expert_ffn_combine) against the FFN followed by the
combine kernel: the same bits in out and y_pool, on the big-tile GEMM Y kernel (bf16,
fp8, mxfp4; where each GEMM Y unit publishes its tile and the kernel's workgroups
combine the tokens once their tiles are done) and on a shape where GEMM Y takes the
general kernel (the combine kernel then follows the FFN). Each case is also held to the
oracle: small shapes on every output element, the full-size skew workload on one token per
pool tile."""
import numpy as np
import pytest
import torch

import combine_moe_dispatch_02_amd as moe
import oracle
from synth import MoEConfig, config_by_name, make_inputs

from _gpu import TOL, dev_inputs, make_layer, out_rows_f64, rel_err, run_layer, say, tile_covering_tokens

pytestmark = pytest.mark.gpu

CASES = [
    MoEConfig("big_both", 1200, 1024, 512, 9, 0, 9, 4, 128),
    MoEConfig("ep_slice", 777, 1024, 256, 12, 3, 5, 4, 128),              # tokens with no local pair
    MoEConfig("fp8_big", 600, 1024, 512, 6, 0, 6, 2, 128, "fp8"),
    MoEConfig("mx_big", 700, 1024, 768, 10, 1, 8, 4, 128, "mxfp4"),
    MoEConfig("general_y", 900, 640, 192, 5, 0, 5, 2, 128),               # GEMM Y on the general kernel
]


def _pair(cfg, streams=False):
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    st = moe.make_streams() if streams else None
    sep = make_layer(cfg)
    a = run_layer(sep, d, st).clone()
    ya = sep.y_pool.clone()
    fused = make_layer(cfg, combine_on_completion=True)
    b = run_layer(fused, d, st).clone()
    return inp, sep, fused, a, ya, b


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_fused_combine_matches_separate(cfg):
    say("combine on completion", cfg.name)
    inp, sep, fused, a, ya, b = _pair(cfg)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # every real pool row of y is the same too (padding rows are unspecified)
    real = (sep.plan.src >= 0).nonzero().squeeze(1)
    assert torch.equal(ya[real].view(torch.int16), fused.y_pool[real].view(torch.int16))
    ref = oracle.moe_layer(inp)
    assert rel_err(out_rows_f64(b), ref.out) <= TOL[cfg.dtype]


def test_fused_combine_two_streams():
    cfg = CASES[1]
    say("combine on completion, two streams", cfg.name)
    inp, _, _, a, _, b = _pair(cfg, streams=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.moe_layer(inp)
    assert rel_err(out_rows_f64(b), ref.out) <= TOL[cfg.dtype]


def test_fused_combine_repeated_calls():
    # the per-tile counters are reset by each call's GEMM A, so back-to-back calls agree
    cfg = CASES[0]
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    fused = make_layer(cfg, combine_on_completion=True)
    say("combine on completion, repeated")
    a = run_layer(fused, d).clone()
    b = run_layer(fused, d).clone()
    c = run_layer(fused, d)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_fused_combine_full_size_skew():
    cfg = config_by_name("zipf_skew")
    say("combine on completion, full size", cfg.name)
    inp, sep, fused, a, ya, b = _pair(cfg)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # against the oracle on the token of every pool tile's last real row (every GEMM Y unit,
    # hence every tile the fused tail waits on, has a compared pair)
    p = oracle.plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    toks = tile_covering_tokens(cfg, inp, p)
    ref = oracle.moe_layer(inp, tokens=toks, p=p)
    err = rel_err(out_rows_f64(b, toks), ref.out)
    print(f"fused combine, {len(toks)} tokens covering all {p.num_tiles} tiles: max-norm rel err {err:.3e}")
    assert err <= TOL[cfg.dtype]
