"""Helpers shared by the GPU parity tests (not a test module)."""
import sys

import numpy as np
import torch

import combine_moe_dispatch_02_amd as moe
import oracle

TOL = {"bf16": 1e-2, "fp8": 3e-2, "mxfp4": 3e-2}


def say(*a):
    """Name the case before each GPU step, flushed, so a dead run still tells which."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def dev_inputs(inp):
    d = {
        "x": inp.x.cuda(),
        "idx": inp.topk_idx.cuda(),
        "w": inp.topk_weights.cuda(),
    }
    if inp.w1 is not None:
        if inp.cfg.dtype in ("fp8", "mxfp4"):
            d["w1"] = inp.w1.view(torch.uint8).cuda()
            d["w2"] = inp.w2.view(torch.uint8).cuda()
            d["w1s"] = inp.w1_scale.cuda()
            d["w2s"] = inp.w2_scale.cuda()
        else:
            d["w1"] = inp.w1.cuda()
            d["w2"] = inp.w2.cuda()
            d["w1s"] = d["w2s"] = None
    return d


def make_layer(shape, **kw):
    return moe.StreamMoE(shape.T, shape.H, shape.I, shape.K, shape.num_local_experts,
                         expert_begin=shape.expert_begin, tile=shape.tile, dtype=shape.dtype, **kw)


def run_layer(layer, d, streams=None):
    if getattr(layer, "_test_w", None) is None:
        layer._test_w = layer.prepare_weights(d["w1"], d["w2"], d["w1s"], d["w2s"])
    w1, w2, w1s, w2s = layer._test_w
    out = layer.forward(d["x"], d["idx"], d["w"], w1, w2, w1s, w2s, streams)
    torch.cuda.synchronize()
    rc = moe.moe_get_error(layer.ws)
    assert rc == 0, f"device error {rc}"
    return out


def assert_plan_equal(plan, op):
    assert np.array_equal(plan.counts.cpu().numpy(), op.counts)
    assert np.array_equal(plan.offsets.cpu().numpy(), op.offsets)
    assert np.array_equal(plan.pos.cpu().numpy(), op.pos)
    assert plan.rows_cap == op.P_cap
    assert np.array_equal(plan.src.cpu().numpy(), op.src)
    assert np.array_equal(plan.tile_expert.cpu().numpy(), op.tile_expert)
    assert int(plan.num_tiles.item()) == op.num_tiles


def out_rows_f64(out, rows=None):
    o = out if rows is None else out[torch.as_tensor(rows, device=out.device)]
    return oracle.bf16_to_f64(o.cpu())


def rel_err(got, ref):
    return oracle.max_norm_rel_err(got, ref)


def tile_covering_tokens(cfg, inp, p, extra=()):
    """Tokens to compare at full size: for every pool tile, the token of its last real row
    (so every tile, and with it every work unit of both GEMMs, has a compared pair), plus the
    first and last token, a token with no local pair and any ``extra``."""
    src = np.asarray(p.src[:p.P]).reshape(-1, cfg.tile)
    pick = set(int(t) for t in extra) | {0, cfg.T - 1}
    for row in src:
        real = row[row >= 0]
        if real.size:
            pick.add(int(real[-1]) // cfg.K)
    idx = inp.topk_idx.numpy()
    local = (idx >= cfg.expert_begin) & (idx < cfg.expert_begin + cfg.num_local_experts)
    if (~local.any(axis=1)).any():
        pick.add(int(np.nonzero(~local.any(axis=1))[0][0]))
    pick.add(int(local.sum(axis=1).argmax()))
    toks = np.array(sorted(pick))
    covered = {int(q) // cfg.tile for t in toks for q in p.pos.reshape(cfg.T, cfg.K)[t] if q >= 0}
    assert covered == set(range(p.num_tiles)), "sample misses a tile"
    return toks
