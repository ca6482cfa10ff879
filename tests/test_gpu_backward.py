"""The backward pass on the GPU against the oracle's exact gradients (bf16 workloads):
dx, the gradient of topk_weights, dW1 and dW2, max-normwise relative error <= 1e-2
each; the training forward keeps G (checked against the oracle's G) and leaves out
bitwise unchanged; the transposed weight re-layout is checked bit for bit.

Small shapes are compared on every element; the skew workload at full size on sampled
tokens (dx, d_topk_weights) and on the weight gradients of sampled experts.

The backward mirrors the forward's per-tile streaming: combine backward raises a ready
flag per dy tile and backward GEMM Y waits on it, so on two streams the two overlap; the
two-stream gradients must equal the one-stream ones bit for bit."""
import random

import numpy as np
import pytest
import torch

import combine_moe_dispatch_02_amd as moe
import oracle
from synth import MoEConfig, config_by_name, make_dout, make_inputs

from _gpu import dev_inputs, make_layer, rel_err, run_layer, say

pytestmark = pytest.mark.gpu

TOL = 1e-2

CASES = [
    MoEConfig("bwd_t128", 300, 512, 512, 6, 0, 6, 2, 128),
    MoEConfig("bwd_t64_ep", 517, 1024, 512, 9, 2, 5, 4, 64),       # experts 2..6 local, ragged tiles
    MoEConfig("bwd_wide", 640, 1536, 1024, 5, 0, 5, 3, 128),
]


def _random_cases(n=6, seed=7331):
    """Seeded random shapes of the training path (bf16, tile 64 or 128, H and I multiples
    of 512, EP slices, uniform or Zipf routing)."""
    rng = random.Random(seed)
    out = []
    for i in range(n):
        E_local = rng.randint(1, 12)
        begin = rng.choice([0, rng.randint(1, 6)])
        E = begin + E_local + rng.choice([0, rng.randint(1, 8)])
        out.append(MoEConfig(f"bwd_rand{i}", rng.randint(1, 400), 512 * rng.randint(1, 3), 512 * rng.randint(1, 2),
                             E, begin, E_local, rng.randint(1, min(8, E)), rng.choice([64, 128]), "bf16",
                             rng.choice(["uniform", "zipf1.2"])))
    return out


CASES += _random_cases()


def expected_t(w):                   # bf16 bits [E, R, K] -> tiled layout of each transpose
    E, R, K = w.shape
    wt = np.ascontiguousarray(w.transpose(0, 2, 1))          # [E, K, R]
    return wt.reshape(E, K // 16, 16, R // 32, 4, 8).transpose(0, 1, 3, 4, 2, 5).reshape(E, K, R)


@pytest.mark.parametrize("shape", [(1, 32, 16), (3, 64, 48), (2, 1024, 512)])
def test_pack_transposed_exact(shape):
    g = torch.Generator().manual_seed(sum(shape) + 7)
    w = torch.randint(-32768, 32767, shape, generator=g, dtype=torch.int16)
    say("pack transposed", shape)
    got = moe.moe_pack_weights_transposed(w.cuda().view(torch.bfloat16))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().view(torch.int16).numpy(), expected_t(w.numpy()))


def _poison(t):
    t.view(torch.uint8).fill_(0xFF)          # NaN as bf16 and fp32


def _train_run(cfg, seed=None, tile_cfg=None, poison=False, streams=None, layer=None):
    inp = make_inputs(cfg) if seed is None else make_inputs(cfg, seed)
    d = dev_inputs(inp)
    if layer is None:
        layer = make_layer(cfg, train=True, cfg=tile_cfg)
    if poison:
        # padding rows of every pool-shaped buffer (pool, y / dy, G / dG, dx_pool) and of h hold
        # NaN; the real rows are all written before they are read
        for t in (layer.pool, layer.y_pool, layer.g_pool, layer.dx_pool):
            _poison(t)
        plan_end = moe.workspace_bytes(cfg.T, cfg.K, cfg.num_local_experts, cfg.tile, layer.pool_rows, 0, "bf16")
        layer.ws.buf[plan_end:].fill_(0xFF)
    w1, w2, _, _ = layer.prepare_weights(d["w1"], d["w2"])
    w1t, w2t = layer.prepare_backward_weights(d["w1"], d["w2"])
    out = layer.forward(d["x"], d["idx"], d["w"], w1, w2, streams=streams).clone()
    g_saved = layer.g_pool.clone()
    dout = make_dout(cfg, inp.seed)
    dx, dw, dW1, dW2 = layer.backward(dout.cuda(), d["w"], w1t, w2t, streams=streams)
    torch.cuda.synchronize()
    assert moe.moe_get_error(layer.ws) == 0
    return inp, d, layer, out, g_saved, dout, dx.clone(), dw.clone(), dW1, dW2


def _bf(t):
    return oracle.bf16_to_f64(t.cpu())


@pytest.mark.parametrize("cfg,poison", [(c, False) for c in CASES] + [(CASES[1], True), (CASES[2], True)],
                         ids=[c.name for c in CASES] + [CASES[1].name + "_poisoned", CASES[2].name + "_poisoned"])
def test_backward_full_compare(cfg, poison):
    # poisoned: the padding rows of the pool, y (then dy), G (then dG), dx_pool and h start as
    # NaN; the weight gradients sum over real rows only, so every result stays finite
    say("backward", cfg.name, "poisoned" if poison else "")
    inp, d, layer, out, g_saved, dout, dx, dw, dW1, dW2 = _train_run(cfg, poison=poison)
    if poison:
        for t in (out, dx, dw, dW1, dW2):
            assert bool(torch.isfinite(t.float()).all())
    # the training forward computes the same out as the inference one
    ref_layer = make_layer(cfg)
    ref_out = run_layer(ref_layer, d)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    g = oracle.moe_layer_backward(inp, dout)

    def err(got, ref):                   # an all-zero reference (no local pair) must be met exactly
        return rel_err(got, ref) if np.abs(ref).max() > 0 else float(np.abs(got).max())

    errs = {
        "dx": err(_bf(dx), g.dx),
        "dw": err(dw.cpu().numpy().astype(np.float64), g.dw),
        "dW1": err(_bf(dW1), g.dW1),
        "dW2": err(_bf(dW2), g.dW2),
    }
    print(cfg.name, {k: f"{v:.2e}" for k, v in errs.items()})
    assert max(errs.values()) <= TOL, errs
    # G as kept by the forward, on the real rows
    src = layer.plan.src.cpu().numpy()
    rows = np.nonzero(src >= 0)[0]
    x = oracle.bf16_to_f64(inp.x)
    ids = inp.topk_idx.numpy().reshape(-1)[src[rows]] - cfg.expert_begin
    G_ref = np.empty((rows.size, 2 * cfg.I))
    for e in np.unique(ids):
        W1 = oracle.bf16_to_f64(inp.w1[e])
        m = ids == e
        G_ref[m] = x[src[rows][m] // cfg.K] @ W1.T
    if rows.size:
        assert rel_err(_bf(g_saved)[rows], G_ref) <= TOL
    # tokens without a local pair get zero gradients
    none_local = ~((inp.topk_idx.numpy() >= cfg.expert_begin)
                   & (inp.topk_idx.numpy() < cfg.expert_begin + cfg.num_local_experts)).any(axis=1)
    assert (_bf(dx)[none_local] == 0).all() and (dw.cpu().numpy()[none_local] == 0).all()


def test_backward_a_pipelines_agree():
    # the data-gradient GEMMs give the same bits with the four-stage ring and with two stages
    cfg = CASES[2]
    say("backward A pipeline depth", cfg.name)
    ring = _train_run(cfg, tile_cfg=moe.TileConfig(0, 0, 0, 0, 0, 4))
    two = _train_run(cfg, tile_cfg=moe.TileConfig(0, 0, 0, 0, 0, 2))
    for i in (6, 7, 8, 9):                        # dx, dw, dW1, dW2
        assert torch.equal(ring[i].view(torch.int32 if ring[i].dtype == torch.float32 else torch.int16),
                           two[i].view(torch.int32 if two[i].dtype == torch.float32 else torch.int16)), i


def _grads_equal(a, b):
    for i in (3, 6, 7, 8, 9):                     # out, dx, dw, dW1, dW2
        assert torch.equal(a[i].view(torch.int32 if a[i].dtype == torch.float32 else torch.int16),
                           b[i].view(torch.int32 if b[i].dtype == torch.float32 else torch.int16)), i


@pytest.mark.parametrize("cfg", [CASES[1], CASES[2]], ids=[CASES[1].name, CASES[2].name])
def test_backward_two_streams(cfg):
    # the backward's mirrored overlap: combine backward on the comm stream raises each dy
    # tile's flag, backward GEMM Y on the compute stream starts on flagged tiles; same bits
    # as one stream, and within tolerance of the oracle's exact gradients
    say("backward two streams", cfg.name)
    one = _train_run(cfg)
    two = _train_run(cfg, streams=moe.make_streams())
    _grads_equal(one, two)
    inp, dout = two[0], two[5]
    g = oracle.moe_layer_backward(inp, dout)
    errs = {"dx": rel_err(_bf(two[6]), g.dx), "dW1": rel_err(_bf(two[8]), g.dW1), "dW2": rel_err(_bf(two[9]), g.dW2)}
    if np.abs(g.dw).max() > 0:
        errs["dw"] = rel_err(two[7].cpu().numpy().astype(np.float64), g.dw)
    print(cfg.name, {k: f"{v:.2e}" for k, v in errs.items()})
    assert max(errs.values()) <= TOL, errs


def test_backward_two_streams_full_size_skew():
    # the skew workload: forward and backward on two streams at the default config give the
    # one-stream bits (those are checked against the oracle by the sampled full-size test)
    cfg = config_by_name("zipf_skew")
    say("backward two streams full size", cfg.name)
    layer = make_layer(cfg, train=True)
    one = _train_run(cfg, layer=layer)
    one = one[:6] + tuple(t.clone() for t in one[6:])
    two = _train_run(cfg, layer=layer, streams=moe.make_streams())
    _grads_equal(one, two)


def test_combine_backward_raises_flags_and_rearms():
    # every real tile's flag equals the call's epoch after combine backward, tiles past the
    # plan's stay 0, and a second call for the same plan (its per-tile counters reset by the
    # first) raises them again with its own epoch and writes the same dy
    cfg = CASES[1]
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    layer = make_layer(cfg, train=True)
    say("combine backward flags", cfg.name)
    moe.moe_plan(d["idx"], layer.plan, layer.ws)
    g = torch.Generator().manual_seed(5)
    y = (torch.randn(layer.y_pool.shape, generator=g) * 0.5).to(torch.bfloat16).cuda()
    dout = make_dout(cfg, inp.seed).cuda()
    nt = int(layer.plan.num_tiles.item())
    dys = []
    for epoch in (11, 12):
        dy = torch.zeros_like(y)
        moe.moe_combine_backward(dout, d["w"], y, layer.plan, dy, layer.dw, epoch, layer.ws)
        torch.cuda.synchronize()
        ready = layer.plan.tile_ready.cpu().numpy().astype(np.int64)
        assert (ready[:nt] == epoch).all() and (ready[nt:] == 0).all()
        dys.append(dy)
    assert moe.moe_get_error(layer.ws) == 0
    assert torch.equal(dys[0].view(torch.int16), dys[1].view(torch.int16))
    # dy rows: w[t,k] * dout[t] rounded once to bf16
    pos = layer.plan.pos.cpu().numpy().reshape(cfg.T, cfg.K)
    t, k = np.nonzero(pos >= 0)
    ref = (inp.topk_weights.numpy()[t, k, None].astype(np.float32)
           * oracle.bf16_to_f64(make_dout(cfg, inp.seed)).astype(np.float32)[t])
    got = dys[0][torch.as_tensor(pos[t, k], device="cuda")].float().cpu().numpy()
    assert np.array_equal(got, torch.from_numpy(ref).to(torch.bfloat16).float().numpy())


def test_ffn_backward_without_combine_backward_times_out():
    # forced from the host: backward GEMM Y waits on an epoch that no combine backward raised,
    # with a 2 ms bound per wait; the call ends with MOE_ERR_TIMEOUT and the workspace is
    # usable again at once
    cfg = CASES[0]
    say("backward forced timeout", cfg.name)
    inp, d, layer, out, g_saved, dout, dx, dw, dW1, dW2 = _train_run(cfg, tile_cfg=moe.TileConfig(0, 0, 2000, 0))
    w1t, w2t = layer.prepare_backward_weights(d["w1"], d["w2"])
    dw1 = torch.empty_like(dW1)
    dw2 = torch.empty_like(dW2)
    moe.moe_expert_ffn_backward(layer.plan, layer.pool, layer.y_pool, layer.g_pool, w1t, w2t, 0xABC, layer.ws,
                                layer.dx_pool, dw1, dw2, layer.cfg)
    torch.cuda.synchronize()
    assert moe.moe_get_error(layer.ws) == moe.layer._abi.MOE_ERR_TIMEOUT
    assert moe.moe_get_error(layer.ws) == 0
    _train_run(cfg, layer=layer)


def test_backward_full_size_skew_sampled():
    cfg = config_by_name("zipf_skew")
    say("backward full size", cfg.name)
    inp, d, layer, out, g_saved, dout, dx, dw, dW1, dW2 = _train_run(cfg)
    idx = inp.topk_idx.numpy()
    counts = np.bincount(idx.reshape(-1), minlength=cfg.num_experts)
    # weight gradients of four experts: the coldest non-empty one, a quartile, the median,
    # and the eighth hottest (a few thousand rows: many K steps of the weight-gradient GEMM)
    nz = np.nonzero(counts)[0]
    order = nz[np.argsort(counts[nz])]
    experts = [int(order[0]), int(order[len(order) // 4]), int(order[len(order) // 2]), int(order[-8])]
    g = oracle.moe_layer_backward(inp, dout, experts=experts)
    for e in experts:
        e1 = rel_err(_bf(dW1[e]), g.dW1[e])
        e2 = rel_err(_bf(dW2[e]), g.dW2[e])
        print(f"expert {e} ({counts[e]} rows): dW1 {e1:.2e} dW2 {e2:.2e}")
        assert e1 <= TOL and e2 <= TOL
    # dx and d_topk_weights of tokens whose pairs all lie in those experts' segments are
    # complete in g; check those tokens
    full = np.isin(idx, experts).all(axis=1)
    part = np.isin(idx, experts)
    toks = np.nonzero(full)[0]
    if toks.size:
        assert rel_err(_bf(dx)[toks], g.dx[toks]) <= TOL
    assert rel_err(dw.cpu().numpy()[part].astype(np.float64), g.dw[part]) <= TOL
    # an expert with no pair has zero weight gradients
    empty = np.nonzero(counts == 0)[0]
    if empty.size:
        assert not bool(dW1[int(empty[0])].float().abs().sum()) and not bool(dW2[int(empty[0])].float().abs().sum())
