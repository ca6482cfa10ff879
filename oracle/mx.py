"""OCP microscaling (MX) codecs for the CPU oracle -- test infrastructure only.

Only tests, the smoke check and the benchmark's CPU-baseline leg import this.

What it follows: the MXFP4 expert-weight format that the pages tie to MI355X MoE
serving (the inference-simulator commit notes, where MXFP4 Quark checkpoints load
on gfx950 only). The pages name the format but not its encoding, so the encoding
is the one the OCP Microscaling Formats (MX) v1.0 specification defines:

* a block is 32 consecutive elements along the contraction dimension sharing one
  scale X = 2^(b - 127) stored as an E8M0 byte b (b = 255 is NaN);
* MXFP4 elements are FP4 E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa
  bit, exponent field 0 subnormal (m * 0.5); no infinities or NaN; largest 6.0;
* MXFP8 elements here are FP8 E4M3 (the oracle's E4M3 codec);
* quantising a block: shared exponent = floor(log2(amax)) - emax_elem, where
  emax_elem is the exponent of the element format's largest normal (2 for E2M1,
  8 for E4M3), clamped to the E8M0 range; each element is then encoded from
  v / X, rounding to nearest even and clamping to the largest magnitude.

Readings where the specification leaves a choice: an all-zero block gets scale
byte 0 (its codes are zero whatever the scale); the clamp of the shared exponent
is to [-127, 127]; quantisation is done on float32 values (the kernels' precision;
the division by a power of two is exact there).
"""
from __future__ import annotations

import numpy as np

from .e4m3 import e4m3_decode, e4m3_encode

MX_BLOCK = 32
E2M1_EMAX = 2
E4M3_EMAX = 8


def _e2m1_from_fields(c: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes 0..15 -> float64, from the bit fields."""
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


# the 16 values, each decoded once from its bit fields
_E2M1_VALUES = _e2m1_from_fields(np.arange(16, dtype=np.int64))


def e2m1_decode(codes) -> np.ndarray:
    """FP4 E2M1 codes (low 4 bits of each entry) -> float64: the bit-field decoding of
    each of the 16 codes, looked up per element."""
    return _E2M1_VALUES[np.asarray(codes).astype(np.intp) & 0xF]


def e8m0_decode(b) -> np.ndarray:
    """E8M0 scale bytes -> float64 2^(b - 127); 255 is NaN."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


def unpack_fp4(packed) -> np.ndarray:
    """uint8 [R, C/2] with the even column in the low nibble -> codes uint8 [R, C]."""
    p = np.asarray(packed, dtype=np.uint8)
    R, Ch = p.shape
    out = np.empty((R, 2 * Ch), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def dequantize_mx_fp4(packed, scale) -> np.ndarray:
    """MXFP4 weights: (packed codes [R, C/2], E8M0 bytes [R, C/32]) -> float64 [R, C]."""
    v = e2m1_decode(unpack_fp4(packed))
    R, C = v.shape
    s = e8m0_decode(scale).reshape(R, C // MX_BLOCK, 1)
    return (v.reshape(R, C // MX_BLOCK, MX_BLOCK) * s).reshape(R, C)


def mx_shared_exponent(amax, emax_elem: int) -> np.ndarray:
    """floor(log2(amax)) - emax_elem, clamped to [-127, 127]; -127 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)                 # amax = f * 2^ex with f in [0.5, 1): floor(log2) = ex - 1
    sh = np.where(amax > 0, ex.astype(np.int64) - 1 - emax_elem, -127)
    return np.clip(sh, -127, 127)


def quantize_mx_e4m3(v) -> tuple:
    """MXFP8 (E4M3) along the last axis: float32 [R, C] -> (codes uint8 [R, C],
    E8M0 bytes uint8 [R, C/32])."""
    v = np.asarray(v, dtype=np.float32)
    R, C = v.shape
    assert C % MX_BLOCK == 0, C
    g = v.reshape(R, C // MX_BLOCK, MX_BLOCK)
    sh = mx_shared_exponent(np.abs(g).max(axis=2), E4M3_EMAX)
    scaled = np.ldexp(g, (-sh)[:, :, None].astype(np.int32)).astype(np.float32)
    codes = e4m3_encode(scaled)
    return codes.reshape(R, C), (sh + 127).astype(np.uint8)


def dequantize_mx_e4m3(codes, scale) -> np.ndarray:
    """(E4M3 codes [R, C], E8M0 bytes [R, C/32]) -> float64 [R, C]."""
    codes = np.asarray(codes)
    R, C = codes.shape
    v = e4m3_decode(codes).reshape(R, C // MX_BLOCK, MX_BLOCK)
    return (v * e8m0_decode(scale)[:, :, None]).reshape(R, C)
