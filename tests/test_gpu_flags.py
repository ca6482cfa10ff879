"""Per-tile ready flags (StreamEP README, "How it works": dispatch signals each pool
tile as it fills and the compute kernels claim ready tiles):
* epochs compare by equality, so the counter's wrap from 2^32-1 to 1 is harmless;
* an FFN whose tiles never become ready ends with MOE_ERR_TIMEOUT instead of hanging
  (forced from the host: the dispatch that would raise the flags is never enqueued);
* running dispatch and the FFN on two streams gives the same bits as one stream."""
import pytest
import torch

import combine_moe_dispatch_02_amd as moe
from synth import config_by_name, MoEConfig, make_inputs

from _gpu import dev_inputs, make_layer, run_layer, say

pytestmark = pytest.mark.gpu


def test_epoch_rollover():
    cfg = config_by_name("tiny")
    d = dev_inputs(make_inputs(cfg))
    layer = make_layer(cfg)
    say("epoch rollover")
    ref = run_layer(layer, d).clone()
    layer.epoch = 0xFFFFFFFE
    a = run_layer(layer, d).clone()
    assert layer.epoch == 0xFFFFFFFF
    b = run_layer(layer, d).clone()
    assert layer.epoch == 1
    assert torch.equal(ref.view(torch.int16), a.view(torch.int16))
    assert torch.equal(ref.view(torch.int16), b.view(torch.int16))


def test_ffn_without_dispatch_times_out():
    cfg = MoEConfig("timeout", 256, 256, 128, 8, 0, 8, 2, 64)
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    layer = make_layer(cfg, cfg=moe.TileConfig(0, 0, 2000, 0))   # 2 ms bound per wait
    say("forced timeout")
    moe.moe_plan(d["idx"], layer.plan, layer.ws)
    # no dispatch: tile_ready stays 0 and never equals epoch 7
    moe.moe_expert_ffn(layer.plan, layer.pool, None, d["w1"], None, d["w2"], None, 7, layer.ws,
                       layer.y_pool, "bf16", layer.cfg)
    torch.cuda.synchronize()
    assert moe.moe_get_error(layer.ws) == moe.layer._abi.MOE_ERR_TIMEOUT
    assert moe.moe_get_error(layer.ws) == 0            # reading clears it
    # the workspace is usable again right away
    run_layer(layer, d)


def test_pool_too_small_is_reported():
    cfg = MoEConfig("small_pool", 256, 256, 128, 8, 0, 8, 2, 64)
    d = dev_inputs(make_inputs(cfg))
    layer = make_layer(cfg, pool_rows=64, cfg=moe.TileConfig(0, 0, 2000, 0))
    say("pool too small")
    layer.forward(d["x"], d["idx"], d["w"], d["w1"], d["w2"])
    torch.cuda.synchronize()
    assert moe.moe_get_error(layer.ws) == moe.layer._abi.MOE_ERR_INVALID


@pytest.mark.parametrize("cfg", [config_by_name("decode"), config_by_name("fp8_weights").with_(name="fp8_4k", T=4096)],
                         ids=["decode", "fp8_4k"])
def test_two_streams_match_one(cfg):
    inp = make_inputs(cfg)
    d = dev_inputs(inp)
    # leave CUs free for the dispatch kernel while the persistent FFN waits on flags
    cus = moe.device_cu_count()
    layer = make_layer(cfg, cfg=moe.TileConfig(0, max(1, cus - 32), 0, 0))
    say("streams", cfg.name)
    one = run_layer(layer, d).clone()
    streams = moe.make_streams()
    two = run_layer(layer, d, streams=streams).clone()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))
