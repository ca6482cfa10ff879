"""Pins of the oracle's e4m3 codec and 1x128 activation quantiser (no GPU).

The codec is checked against the OCP E4M3 definition at named points, against
torch's own float8_e4m3fn conversion (a library routine written independently
of the oracle), and exhaustively over all 256 codes.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3_decode, e4m3_encode


def test_named_values():
    v = oracle.E4M3_VALUES
    assert v[0x00] == 0.0
    assert v[0x01] == 2.0 ** -9            # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert v[0x08] == 2.0 ** -6            # smallest normal
    assert v[0x38] == 1.0                  # exponent field 7 = bias
    assert v[0x7E] == 448.0                # largest finite
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0xB8] == -1.0
    assert v[0xFE] == -448.0


def test_decode_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(np.arange(256, dtype=np.uint8))
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.signbit(got[~both_nan]), np.signbit(ref[~both_nan]))


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), codes)


def test_encode_ties_go_to_even_mantissa():
    pos = oracle.E4M3_VALUES[:127]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)  # exact in fp32
    got = e4m3_encode(mids)
    lo = np.arange(126)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    # just above / below a midpoint goes to the nearer neighbour
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    assert np.array_equal(e4m3_encode(up), (lo + 1).astype(np.uint8))
    assert np.array_equal(e4m3_encode(dn), lo.astype(np.uint8))


def test_encode_matches_torch_inside_range():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 40,
        rng.uniform(-448, 448, 100_000).astype(np.float32),
        (rng.standard_normal(50_000) * 2.0 ** -8).astype(np.float32),   # subnormal range
    ])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(v), ref)


def test_encode_saturates_and_keeps_sign_of_zero():
    v = np.array([448.0, 460.0, 464.0, 1e6, -500.0, -0.0, -1e-12, 1e-12, 0.0], dtype=np.float32)
    assert e4m3_encode(v).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00, 0x00]


def test_encode_rejects_non_finite():
    with pytest.raises(ValueError):
        e4m3_encode(np.array([np.inf], dtype=np.float32))


# ------------------------- 1x128 group quantiser ---------------------------- #
def test_group_quantiser_error_bound_and_extremes():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[3, 128:256] = 0.0                                   # an all-zero group
    codes, s = oracle.quantize_groups(x)
    assert codes.shape == x.shape and s.shape == (64, 4)
    assert s[3, 1] == 1.0 and (codes[3, 128:256] == 0).all()
    g = x.reshape(64, 4, 128)
    amax = np.abs(g).max(axis=2)
    assert np.array_equal(s[amax > 0], (amax / np.float32(448))[amax > 0])
    # the group's largest magnitude lands on +-448
    c = codes.reshape(64, 4, 128)
    arg = np.abs(g).argmax(axis=2)
    top = np.take_along_axis(c, arg[:, :, None], axis=2)[..., 0]
    assert np.all((top[amax > 0] & 0x7F) == 0x7E)
    # reconstruction error: half a mantissa step of 3 bits for normals,
    # half the subnormal step (2^-10 in scaled units) below 2^-6
    deq = oracle.dequantize_groups(codes, s).reshape(64, 4, 128)
    scaled = np.abs(g) / s[:, :, None]
    err = np.abs(deq - g) / s[:, :, None]
    bound = np.where(scaled >= 2.0 ** -6, scaled * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_group_scales_follow_rows_and_groups():
    # each (row, group) gets its own scale: row r, group j holds the value 448 * (r+1) * 2^j
    R, G = 3, 4
    x = np.zeros((R, 128 * G), dtype=np.float32)
    for r in range(R):
        for j in range(G):
            x[r, j * 128] = 448.0 * (r + 1) * 2.0 ** j
    codes, s = oracle.quantize_groups(x)
    for r in range(R):
        for j in range(G):
            assert s[r, j] == (r + 1) * 2.0 ** j
            assert codes[r, j * 128] == 0x7E


def test_weight_block_scales_orientation():
    # codes all 1.0; block (br, bc) scale = 2^br * 3^bc -> value at (r, c) = scale[r//128, c//128]
    R, C = 256, 384
    codes = np.full((R, C), 0x38, dtype=np.uint8)
    sc = np.array([[2.0 ** br * 3.0 ** bc for bc in range(3)] for br in range(2)], dtype=np.float32)
    w = oracle.dequantize_blocks(codes, sc)
    assert w[0, 0] == 1.0 and w[127, 127] == 1.0
    assert w[128, 0] == 2.0 and w[0, 128] == 3.0 and w[255, 383] == 18.0
