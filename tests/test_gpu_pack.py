"""moe_pack_weights moves values into MFMA fragment order exactly as include/moe355.h
states it; checked bit for bit against a NumPy reshape/transpose of that statement."""
import numpy as np
import pytest
import torch

import combine_moe_dispatch_02_amd as moe

from _gpu import say

pytestmark = pytest.mark.gpu


def expected_bf16(w):            # w: uint16 [E, R, K]
    E, R, K = w.shape
    # value (e, rb*16 + r, kb*32 + 8*q + i) sits at tile (rb, kb), lane q*16 + r, element i
    return w.reshape(E, R // 16, 16, K // 32, 4, 8).transpose(0, 1, 3, 4, 2, 5).reshape(E, R, K)


def expected_fp8(w):             # w: uint8 [E, R, K]
    E, R, K = w.shape
    # value (e, rb*16 + r, kb*128 + 32*q + 16*h + i) at tile (rb, kb), half h, lane q*16 + r, byte i
    return w.reshape(E, R // 16, 16, K // 128, 4, 2, 16).transpose(0, 1, 3, 5, 4, 2, 6).reshape(E, R, K)


@pytest.mark.parametrize("shape", [(1, 16, 32), (3, 48, 96), (2, 3072, 4096)])
def test_pack_bf16_exact(shape):
    g = torch.Generator().manual_seed(sum(shape))
    w = torch.randint(-32768, 32767, shape, generator=g, dtype=torch.int16)
    say("pack bf16", shape)
    got = moe.moe_pack_weights(w.cuda().view(torch.bfloat16), "bf16")
    torch.cuda.synchronize()
    ref = expected_bf16(w.numpy().view(np.uint16))
    assert np.array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), ref)


@pytest.mark.parametrize("shape", [(1, 16, 128), (4, 32, 384)])
def test_pack_fp8_exact(shape):
    g = torch.Generator().manual_seed(sum(shape) + 1)
    w = torch.randint(0, 255, shape, generator=g, dtype=torch.uint8)
    say("pack fp8", shape)
    got = moe.moe_pack_weights(w.cuda(), "fp8")
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), expected_fp8(w.numpy()))


def expected_mx_codes(w):        # w: uint8 [E, R, K/2] (two e2m1 codes per byte)
    E, R, Kh = w.shape
    # byte (e, rb*16 + r, kb*64 + 16*q + i) sits at tile (rb, kb), lane q*16 + r, byte i
    return w.reshape(E, R // 16, 16, Kh // 64, 4, 16).transpose(0, 1, 3, 4, 2, 5).reshape(E, R, Kh)


def expected_mx_scales(s):       # s: uint8 [E, R, K/32]
    E, R, KB = s.shape
    # scale (e, rb*16 + r, kb*4 + q) sits at tile (rb, kb), byte q*16 + r
    return s.reshape(E, R // 16, 16, KB // 4, 4).transpose(0, 1, 3, 4, 2).reshape(E, R, KB)


@pytest.mark.parametrize("shape", [(1, 16, 128), (3, 48, 384), (2, 3072, 4096)])
def test_pack_mxfp4_codes_and_scales_exact(shape):
    E, R, K = shape
    g = torch.Generator().manual_seed(sum(shape) + 2)
    w = torch.randint(0, 256, (E, R, K // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    s = torch.randint(0, 256, (E, R, K // 32), generator=g, dtype=torch.int32).to(torch.uint8)
    say("pack mxfp4", shape)
    got_w = moe.moe_pack_weights(w.cuda(), "mxfp4")
    got_s = moe.moe_pack_mx_scales(s.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(got_w.cpu().numpy(), expected_mx_codes(w.numpy()))
    assert np.array_equal(got_s.cpu().numpy(), expected_mx_scales(s.numpy()))


def test_pack_rejects_bad_shapes():
    w = torch.zeros(1, 24, 32, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_pack_weights(w, "bf16")
    s = torch.zeros(1, 16, 3, dtype=torch.uint8, device="cuda")   # K = 96: not whole 128-K tiles
    with pytest.raises(moe.MoeError):
        moe.moe_pack_mx_scales(s)
