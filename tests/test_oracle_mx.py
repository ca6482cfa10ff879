"""Pins of the oracle's MX codecs and of its mxfp4 layer (no GPU).

* E8M0 decoding against torch's float8_e8m0fnu conversion (a library routine);
* E2M1 decoding against the value table of the OCP MX specification
  (tests/golden/e2m1_values.json) and its sign symmetry;
* the fp4 nibble order on a hand-worked byte, and the MXFP4 dequantiser against
  an element-by-element loop;
* the shared-exponent rule on closed cases (powers of two, saturation, zero,
  the clamps), and the MXFP8 quantiser against a brute-force nearest-value
  search over the 253 finite E4M3 values, plus its error bound;
* the mxfp4 layer on grid-exact operands equals the bf16 layer up to h's
  rounding, which is bounded by half an E4M3 mantissa step.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import MoEConfig, MoEInputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e8m0_decode_matches_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.e8m0_decode(b.numpy())
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_e2m1_decode_matches_spec_table():
    g = json.load(open(os.path.join(GOLDEN, "e2m1_values.json")))
    vals = oracle.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == g["values"]
    assert np.array_equal(vals[8:], -vals[:8])
    assert math.copysign(1.0, vals[8]) == -1.0          # code 8 is -0
    # only the low nibble of an entry counts
    assert np.array_equal(oracle.e2m1_decode(np.arange(16) + 0x30), vals)


def test_fp4_nibble_order_hand_worked():
    # byte 0x21: low nibble 1 (column 0) = 0.5, high nibble 2 (column 1) = 1.0;
    # byte 0xF8: column 2 = code 8 = -0, column 3 = code 15 = -6
    codes = oracle.unpack_fp4(np.array([[0x21, 0xF8]], dtype=np.uint8))
    assert codes.tolist() == [[1, 2, 8, 15]]


def test_mx_fp4_dequantize_elementwise():
    rng = np.random.default_rng(3)
    R, C = 3, 96
    packed = rng.integers(0, 256, size=(R, C // 2)).astype(np.uint8)
    scale = rng.integers(120, 135, size=(R, C // 32)).astype(np.uint8)
    got = oracle.dequantize_mx_fp4(packed, scale)
    table = json.load(open(os.path.join(GOLDEN, "e2m1_values.json")))["values"]
    for r in range(R):
        for c in range(C):
            byte = int(packed[r, c // 2])
            code = (byte >> 4) if c % 2 else (byte & 15)
            mag = table[code & 7]
            v = (-mag if code & 8 else mag) * 2.0 ** (int(scale[r, c // 32]) - 127)
            assert got[r, c] == v, (r, c)


@pytest.mark.parametrize("amax,emax,want", [
    (1.0, 8, -8), (2.0 ** 10, 8, 2), (2.0 ** 10 * 1.999, 8, 2), (500.0, 8, 0),
    (6.0, 2, 0), (7.9, 2, 0), (0.75, 2, -3), (0.0, 8, -127),
    (2.0 ** -125, 8, -127), (2.0 ** -119, 8, -127), (2.0 ** -118, 8, -126),
    (3.0e38, 8, 119), (3.0e38, 2, 125)])
def test_shared_exponent_closed_cases(amax, emax, want):
    assert int(oracle.mx_shared_exponent(np.float64(amax), emax)) == want


def test_mx_e4m3_special_blocks():
    x = np.zeros((3, 64), dtype=np.float32)
    x[0, 5] = 2.0 ** 12                  # amax a power of two -> scaled to exactly 256
    x[0, 6] = -3.0
    x[0, 40] = 500.0                     # second block: 500 saturates to 448 at scale 1
    x[0, 41] = 1.0
    x[1, :32] = 0.0                      # an all-zero block
    x[1, 32:] = np.linspace(-1, 1, 32, dtype=np.float32)
    codes, s = oracle.quantize_mx_e4m3(x)
    assert s[0, 0] == 127 + 4 and codes[0, 5] == 0x78
    assert oracle.e4m3_decode(codes[0, 6]) * 2.0 ** 4 == -2.0 ** 4 * 0.1875
    assert s[0, 1] == 127 and codes[0, 40] == 0x7E and codes[0, 41] == 0x38
    assert s[1, 0] == 0 and not codes[1, :32].any()
    assert s[1, 1] == 127 - 8            # amax 1 -> 2^-8
    assert s[2, 0] == 0 and s[2, 1] == 0


def _nearest_even_code(a: float) -> int:
    """Brute force: the non-negative E4M3 code nearest to a (ties: even code), saturating."""
    pos = oracle.E4M3_VALUES[:127]
    if a >= pos[-1]:
        return 126
    d = np.abs(pos - a)
    best = np.flatnonzero(d == d.min())
    return int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])


def test_mx_e4m3_matches_brute_force_and_error_bound():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((6, 96)) * np.exp2(rng.integers(-20, 20, size=(6, 1)))).astype(np.float32)
    x[2, 7] = 0.0
    codes, s = oracle.quantize_mx_e4m3(x)
    for r in range(6):
        for b in range(3):
            blk = x[r, 32 * b:32 * b + 32].astype(np.float64)
            sh = int(s[r, b]) - 127
            assert math.floor(math.log2(np.abs(blk).max())) - 8 == sh
            for i, v in enumerate(blk):
                want = _nearest_even_code(abs(v) * 2.0 ** -sh) | (0x80 if math.copysign(1.0, v) < 0 else 0)
                assert codes[r, 32 * b + i] == want, (r, b, i)
    deq = oracle.dequantize_mx_e4m3(codes, s)
    for r in range(6):
        for b in range(3):
            X = 2.0 ** (int(s[r, b]) - 127)
            for i in range(32):
                v = float(x[r, 32 * b + i])
                a = abs(v) / X
                if a > 448:                                   # saturation: at most 512 - 448
                    assert abs(deq[r, 32 * b + i] - v) <= 64 * X
                    continue
                ulp = 2.0 ** (max(math.floor(math.log2(a)), -6) - 3) if a > 0 else 2.0 ** -9
                assert abs(deq[r, 32 * b + i] - v) <= 0.5 * ulp * X


def test_mxfp4_layer_on_exact_operands_equals_bf16_layer_up_to_h_rounding():
    # x: E4M3 values with 256 (code 0x78) in every block, so MXFP8 keeps them exactly at
    # scale 1; weights: E2M1 codes with E8M0 bytes 124..127 (bf16-exact products), so
    # GEMM A sees the same operands on both paths and only h's quantisation differs.
    T, H, I, E = 6, 64, 64, 2
    cfg = MoEConfig("exact_mx", T, H, I, E, 0, E, 1, 4, "mxfp4")
    rng = np.random.default_rng(5)
    codes = rng.integers(0x20, 0x70, size=(T, H)).astype(np.uint8)
    codes[:, 0] = 0x78
    codes[:, 32] = 0xF8
    x = torch.from_numpy(oracle.e4m3_decode(codes).astype(np.float32)).to(torch.bfloat16)
    w1p = rng.integers(0, 256, size=(E, 2 * I, H // 2)).astype(np.uint8)
    w2p = rng.integers(0, 256, size=(E, H, I // 2)).astype(np.uint8)
    w1s = rng.integers(118, 122, size=(E, 2 * I, H // 32)).astype(np.uint8)
    w2s = rng.integers(118, 122, size=(E, H, I // 32)).astype(np.uint8)
    idx = torch.tensor([[0], [1], [0], [1], [1], [0]], dtype=torch.int32)
    w = torch.ones(T, 1)
    inp = MoEInputs(cfg, 0, x, idx, w, torch.from_numpy(w1p), torch.from_numpy(w1s),
                    torch.from_numpy(w2p), torch.from_numpy(w2s))
    xq, xs = oracle.quantize_mx_e4m3(oracle.bf16_to_f64(x).astype(np.float32))
    assert np.array_equal(xq, codes) and (xs == 127).all()
    w1b = torch.from_numpy(np.stack([oracle.dequantize_mx_fp4(w1p[e], w1s[e]) for e in range(E)])).to(torch.bfloat16)
    w2b = torch.from_numpy(np.stack([oracle.dequantize_mx_fp4(w2p[e], w2s[e]) for e in range(E)])).to(torch.bfloat16)
    assert np.array_equal(oracle.bf16_to_f64(w1b[0]), oracle.dequantize_mx_fp4(w1p[0], w1s[0]))
    inpb = MoEInputs(cfg.with_(dtype="bf16"), 0, x, idx, w, w1b, None, w2b, None)
    om = oracle.moe_layer(inp).out
    ob = oracle.moe_layer(inpb).out
    err = oracle.max_norm_rel_err(om, ob)
    assert 0 < err < 2.0 ** -4
