"""A2 and A5 on the GPU, without the FFN:
* dispatch writes exactly the oracle's pool rows (bf16 bits; e4m3 codes and fp32 group
  scales; MXFP8 e4m3 codes and E8M0 block scales; the scales read back from the
  tile-major words the ABI documents), leaves poisoned padding rows alone, and raises
  every tile's ready flag;
* with identity experts (y_pool = pool) combine returns sum_k w_k x_t, and with
  K = 1, w = 1 the dispatch -> combine round trip is bit-exact."""
import numpy as np
import pytest
import torch

import combine_moe_dispatch_02_amd as moe
import oracle
from synth import MoEConfig, config_by_name, make_inputs

from _gpu import say

pytestmark = pytest.mark.gpu

POISON = 0x7FC1  # a bf16 NaN pattern


def scale_rows(words, rows, tile, per_row):
    """Scale words stored tile-major (row p's word for group g at word
    (p // tile * groups + g) * tile + p % tile, 4 bytes each) -> [rows][per_row] in row
    order: fp32 words for fp8, the 4 E8M0 bytes of each word for mxfp4."""
    w = words.cpu().numpy().reshape(-1)
    unit = 1 if w.dtype == np.float32 else 4
    groups = per_row // unit
    w = w[: rows * per_row].reshape(rows // tile, groups, tile, unit)
    return w.transpose(0, 2, 1, 3).reshape(rows, per_row)


def plan_and_dispatch(inp, epoch=5, fp8=False, dtype=None):
    """Plan and dispatch; pool_s comes back in row order (see scale_rows)."""
    c = inp.cfg
    dtype = dtype or ("fp8" if fp8 else "bf16")
    plan = moe.Plan.allocate(c.T, c.K, c.expert_begin, c.num_local_experts, c.tile)
    ws = moe.Workspace(c.T, c.K, c.num_local_experts, c.tile)
    rows = plan.rows_cap
    if dtype == "fp8":
        pool = torch.full((rows, c.H), 0x7F, dtype=torch.uint8, device="cuda")
        pool_s = torch.full((rows, c.H // 128), -1.0, dtype=torch.float32, device="cuda")
    elif dtype == "mxfp4":
        pool = torch.full((rows, c.H), 0x7F, dtype=torch.uint8, device="cuda")
        pool_s = torch.full((rows, (c.H + 127) // 128 * 4), 0xFF, dtype=torch.uint8, device="cuda")
    else:
        pool = torch.full((rows, c.H), POISON, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        pool_s = None
    x = inp.x.cuda()
    moe.moe_plan(inp.topk_idx.cuda(), plan, ws)
    moe.moe_dispatch(x, plan, pool, pool_s, epoch, ws, dtype)
    torch.cuda.synchronize()
    assert moe.moe_get_error(ws) == 0
    if pool_s is not None:
        pool_s = scale_rows(pool_s, rows, c.tile, pool_s.shape[1])
    return plan, ws, pool, pool_s


SMALL = [
    config_by_name("tiny"),
    config_by_name("decode"),
    MoEConfig("ragged", 333, 392, 64, 11, 3, 6, 3, 32),      # H not a multiple of 512 chunks
    MoEConfig("ep_small", 700, 7168, 64, 64, 0, 8, 8, 128),   # two row segments per lane
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_dispatch_bf16_rows_exact(cfg):
    inp = make_inputs(cfg, weights=False)
    say("dispatch bf16", cfg.name)
    plan, ws, pool, _ = plan_and_dispatch(inp)
    op = oracle.plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    rows, payload = oracle.dispatch(inp.x, op, fp8=False)
    got = pool.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got[rows], payload)
    pad = np.setdiff1d(np.arange(op.P_cap), rows)
    assert (got[pad] == POISON).all()                       # nothing written outside real rows
    ready = plan.tile_ready.cpu().numpy()
    assert (ready[: op.num_tiles] == 5).all() and (ready[op.num_tiles:] == 0).all()


def test_dispatch_full_size_rows_match_source_token():
    # at the largest workload: every real pool row equals its source token's row
    cfg = config_by_name("zipf_skew")
    inp = make_inputs(cfg, weights=False)
    say("dispatch bf16 full size", cfg.name)
    plan, ws, pool, _ = plan_and_dispatch(inp)
    src = plan.src.long()
    real = src >= 0
    tok = torch.where(real, src // cfg.K, torch.zeros_like(src))
    x = inp.x.cuda()
    same = (pool.view(torch.int16)[real] == x.view(torch.int16)[tok[real]]).all()
    assert bool(same)
    assert int(real.sum()) == cfg.T * cfg.K
    nt = int(plan.num_tiles.item())
    assert bool((plan.tile_ready[:nt] == 5).all())


FP8 = [
    MoEConfig("fp8_small", 300, 512, 128, 10, 0, 10, 4, 64, "fp8"),
    MoEConfig("fp8_ragged", 129, 1152, 128, 7, 2, 4, 3, 128, "fp8"),
]


@pytest.mark.parametrize("cfg", FP8, ids=[c.name for c in FP8])
def test_dispatch_fp8_codes_and_scales_exact(cfg):
    inp = make_inputs(cfg, weights=False)
    # an all-zero group and a row with a tiny and a huge value
    inp.x[3, 128:256] = 0
    inp.x[5, 7] = 3.0e-38
    inp.x[5, 9] = -2.5e30
    say("dispatch fp8", cfg.name)
    plan, ws, pool, pool_s = plan_and_dispatch(inp, fp8=True)
    op = oracle.plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    rows, (codes, scales) = oracle.dispatch(inp.x, op, fp8=True)
    assert np.array_equal(pool.cpu().numpy()[rows], codes)
    assert np.array_equal(pool_s[rows, : scales.shape[1]], scales)


def test_dispatch_fp8_full_size_sampled_rows():
    cfg = config_by_name("fp8_weights")
    inp = make_inputs(cfg, weights=False)
    say("dispatch fp8 full size", cfg.name)
    plan, ws, pool, pool_s = plan_and_dispatch(inp, fp8=True)
    src = plan.src.cpu().numpy()
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(np.nonzero(src >= 0)[0], 256, replace=False))
    codes, scales = oracle.token_rows(inp.x, True, src[rows] // cfg.K)
    assert np.array_equal(pool.cpu().numpy()[rows], codes)
    assert np.array_equal(pool_s[rows, : scales.shape[1]], scales)


MX = [
    MoEConfig("mx_small", 300, 512, 128, 10, 0, 10, 4, 64, "mxfp4"),
    MoEConfig("mx_ragged", 129, 1184, 128, 7, 2, 4, 3, 128, "mxfp4"),    # 37 blocks: a partial lane sweep
]


@pytest.mark.parametrize("cfg", MX, ids=[c.name for c in MX])
def test_dispatch_mxfp8_codes_and_scales_exact(cfg):
    inp = make_inputs(cfg, weights=False)
    inp.x[3, 32:64] = 0                                       # an all-zero block
    inp.x[5, 7] = -2.5e30                                     # a huge value
    inp.x[5, 40] = 256.0                                      # amax exactly a power of two
    inp.x[5, 41:64] = 0
    inp.x[6, 64:96] = torch.linspace(-1e-39, 1e-39, 32)      # bf16 subnormals only: clamped scale
    inp.x[7, :32] = 3.0e-38
    say("dispatch mxfp8", cfg.name)
    plan, ws, pool, pool_s = plan_and_dispatch(inp, dtype="mxfp4")
    op = oracle.plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    rows, (codes, scales) = oracle.dispatch(inp.x, op, "mxfp4")
    assert np.array_equal(pool.cpu().numpy()[rows], codes)
    assert np.array_equal(pool_s[rows, : scales.shape[1]], scales)
    pad = np.setdiff1d(np.arange(op.P_cap), rows)
    assert (pool_s[pad] == 0xFF).all()
    assert (pool_s[rows, scales.shape[1]:] == 0xFF).all()       # the last word's bytes past H/32


def test_dispatch_mxfp8_full_size_sampled_rows():
    cfg = config_by_name("mxfp4")
    inp = make_inputs(cfg, weights=False)
    say("dispatch mxfp8 full size", cfg.name)
    plan, ws, pool, pool_s = plan_and_dispatch(inp, dtype="mxfp4")
    src = plan.src.cpu().numpy()
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(np.nonzero(src >= 0)[0], 256, replace=False))
    codes, scales = oracle.token_rows(inp.x, "mxfp4", src[rows] // cfg.K)
    assert np.array_equal(pool.cpu().numpy()[rows], codes)
    assert np.array_equal(pool_s[rows, : scales.shape[1]], scales)


@pytest.mark.parametrize("cfg", [config_by_name("tiny"), MoEConfig("ident", 515, 256, 64, 12, 4, 5, 4, 16)],
                         ids=["tiny", "ident_nonlocal"])
def test_identity_expert_combine(cfg):
    inp = make_inputs(cfg, weights=False)
    say("identity combine", cfg.name)
    plan, ws, pool, _ = plan_and_dispatch(inp)
    out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device="cuda")
    w = inp.topk_weights.cuda()
    moe.moe_combine(pool, w, plan, out)
    torch.cuda.synchronize()
    got = oracle.bf16_to_f64(out.cpu())
    op = oracle.plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    local = op.pos.reshape(cfg.T, cfg.K) >= 0
    x = oracle.bf16_to_f64(inp.x)
    ref = oracle.combine(np.repeat(x[:, None, :], cfg.K, axis=1), inp.topk_weights, local)
    # one fp32 accumulation and one bf16 rounding: within half a bf16 ulp plus fp32 noise
    tol = np.abs(ref) * 2.0 ** -8 + 1e-30
    assert (np.abs(got - ref) <= tol).all()
    assert (got[~local.any(axis=1)] == 0).all()


def test_permutation_round_trip_k1_exact():
    cfg = MoEConfig("perm", 1000, 512, 64, 7, 0, 7, 1, 32)
    inp = make_inputs(cfg, weights=False)
    say("round trip K=1")
    plan, ws, pool, _ = plan_and_dispatch(inp)
    out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(pool, torch.ones(cfg.T, 1, device="cuda"), plan, out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), inp.x.view(torch.int16))
