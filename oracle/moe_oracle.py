"""CPU oracle of the MoE dispatch -> expert FFN -> combine path -- test infrastructure only.

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
module. The GPU library never calls it and shares no code with it.

What it follows (StreamEP README, section "How it works"):

* Pool-layout dispatch: every routed (token, k) pair lands in an expert-major,
  tile-padded pool, so the pool is the grouped GEMM's input as it stands.
* The forward grouped GEMMs "A" (w1, gate|up, then the activation) and "Y" (w2)
  run over the pool, one expert segment at a time.
* Combine sends each token's expert outputs back, where they are reduced with
  that token's ``topk_weights`` (README usage sample: ``topk_idx``,
  ``topk_weights``, ``w1_local``, ``w2_local``).

Readings where the page is silent (each is the plainest one the rest supports):

1. Inside an expert's segment, pairs keep the order of their flat pair id
   q = t*K + k (a stable counting sort).
2. A segment is padded to ceil(count/tile)*tile rows; an empty expert gets no rows.
3. Ids outside [expert_begin, expert_begin + E_local), and -1, are not local:
   pos = -1, not counted, and their weight is dropped (no renormalisation).
4. w1[e] is [2I, H] with rows 0..I-1 the gate and rows I..2I-1 the up
   projection; w2[e] is [H, I]. h = silu(gate) * up, silu(z) = z / (1 + e^-z).
5. fp8: activations are quantised per 1x128 group of the contraction dim
   (H for x, I for h) with scale = amax / 448 in fp32 (1 when amax = 0),
   codes = e4m3(value / scale); weights are code * block scale (128x128).
   The quantisation decisions are taken in fp32, the kernels' precision.
6. combine: out[t] = sum over local k, ascending, of w[t,k] * y(t,k);
   a token with no local pair gets a zero row.
7. mxfp4 (weights MXFP4, the format the pages tie to MI355X MoE serving):
   weights are E2M1 codes times an E8M0 scale per 1x32 block along K, as the
   OCP MX specification defines them (oracle/mx.py); activations (x, and h
   before GEMM Y) are MXFP8: E4M3 codes with an E8M0 scale per 1x32 block,
   quantised per that specification in float32.

Arithmetic: float64 on the dequantised values (bf16 -> float is exact), with
no intermediate rounding except the fp8 activation quantisation of reading 5.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .e4m3 import e4m3_decode, e4m3_encode
from .mx import dequantize_mx_e4m3, dequantize_mx_fp4, quantize_mx_e4m3

GROUP = 128  # fp8 activation group / weight block edge


# --------------------------------------------------------------------------- #
# host views of the inputs
# --------------------------------------------------------------------------- #
def _np(t) -> np.ndarray:
    """A torch CPU tensor or numpy array -> numpy array (no copy when possible)."""
    if isinstance(t, np.ndarray):
        return t
    return t.detach().cpu().numpy()


def bf16_bits(t) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of a torch bfloat16 tensor."""
    import torch  # only for the dtype-preserving view; arithmetic stays in numpy

    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(t) -> np.ndarray:
    """bf16 tensor -> float64: the 16 bits are the top half of an IEEE binary32."""
    b = bf16_bits(t).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _mode(dtype) -> str:
    """Activation/weight format: "bf16", "fp8" or "mxfp4" (a bool means fp8 or bf16)."""
    if isinstance(dtype, (bool, np.bool_)):
        return "fp8" if dtype else "bf16"
    if dtype not in ("bf16", "fp8", "mxfp4"):
        raise ValueError(dtype)
    return dtype


def fp8_codes(t) -> np.ndarray:
    import torch

    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


# --------------------------------------------------------------------------- #
# A1: placement plan
# --------------------------------------------------------------------------- #
def pool_rows_bound(T: int, K: int, E_local: int, tile: int) -> int:
    """Rows any plan can need: ceil(c/tile)*tile <= c + tile - 1 summed over experts,
    rounded down to a whole tile (pool sizes are whole tiles)."""
    return ((T * K + E_local * (tile - 1)) // tile) * tile


@dataclass
class OraclePlan:
    counts: np.ndarray       # int32 [E_local]
    offsets: np.ndarray      # int32 [E_local + 1]; offsets[E_local] = P
    pos: np.ndarray          # int32 [T*K]; pool row of pair q, -1 if not local
    src: np.ndarray          # int32 [P_cap]; pair id of pool row p, -1 for padding/unused
    tile_expert: np.ndarray  # int32 [P_cap / tile]; local expert of tile i, -1 past num_tiles
    num_tiles: int
    P: int                   # pool rows in use
    P_cap: int               # allocation bound
    T: int
    K: int
    tile: int


def plan(topk_idx, expert_begin: int, E_local: int, tile: int) -> OraclePlan:
    """Expert-major, tile-padded placement of the local (token, k) pairs."""
    ids = _np(topk_idx).astype(np.int64)
    T, K = ids.shape
    flat = ids.reshape(-1)
    q_all = np.arange(T * K, dtype=np.int64)
    local = (flat >= expert_begin) & (flat < expert_begin + E_local)
    q = q_all[local]
    e = flat[local] - expert_begin

    counts = np.bincount(e, minlength=E_local).astype(np.int64)
    padded = (counts + tile - 1) // tile * tile
    offsets = np.zeros(E_local + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    P = int(offsets[-1])
    P_cap = pool_rows_bound(T, K, E_local, tile)
    assert P <= P_cap

    # reading 1: stable in q inside each expert
    order = np.argsort(e, kind="stable")
    q_sorted = q[order]
    e_sorted = e[order]
    first = np.zeros(E_local, dtype=np.int64)
    first[1:] = np.cumsum(counts)[:-1]
    rank = np.arange(q_sorted.size, dtype=np.int64) - first[e_sorted]

    pos = np.full(T * K, -1, dtype=np.int64)
    pos[q_sorted] = offsets[e_sorted] + rank
    src = np.full(P_cap, -1, dtype=np.int64)
    src[pos[q_sorted]] = q_sorted

    ntiles_cap = P_cap // tile
    tile_expert = np.full(ntiles_cap, -1, dtype=np.int64)
    for ex in range(E_local):
        tile_expert[offsets[ex] // tile: offsets[ex + 1] // tile] = ex

    i32 = lambda a: a.astype(np.int32)  # noqa: E731
    return OraclePlan(i32(counts), i32(offsets), i32(pos), i32(src), i32(tile_expert),
                      P // tile, P, P_cap, T, K, tile)


# --------------------------------------------------------------------------- #
# fp8 activation groups (reading 5)
# --------------------------------------------------------------------------- #
def quantize_groups(v) -> tuple:
    """float32 [R, C] -> (e4m3 codes uint8 [R, C], scales float32 [R, C/128])."""
    v = np.asarray(v, dtype=np.float32)
    R, C = v.shape
    assert C % GROUP == 0, C
    g = v.reshape(R, C // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = e4m3_encode((g / scale[:, :, None]).astype(np.float32))
    return codes.reshape(R, C), scale


def dequantize_groups(codes, scale) -> np.ndarray:
    """(codes [R, C], scales [R, C/128]) -> float64 [R, C]."""
    codes = np.asarray(codes)
    R, C = codes.shape
    v = e4m3_decode(codes).reshape(R, C // GROUP, GROUP)
    return (v * np.asarray(scale, dtype=np.float64)[:, :, None]).reshape(R, C)


def dequantize_blocks(codes, scale) -> np.ndarray:
    """Weights: (codes [R, C], block scales [R/128, C/128]) -> float64 [R, C]."""
    codes = np.asarray(codes)
    R, C = codes.shape
    v = e4m3_decode(codes).reshape(R // GROUP, GROUP, C // GROUP, GROUP)
    s = np.asarray(scale, dtype=np.float64)[:, None, :, None]
    return (v * s).reshape(R, C)


# --------------------------------------------------------------------------- #
# A2: what dispatch must place
# --------------------------------------------------------------------------- #
def token_rows(x, fp8, tokens: Optional[np.ndarray] = None):
    """Activation rows as the expert GEMM consumes them (``fp8``: a format name or bool).

    bf16: float64 copy of x. fp8: (codes, fp32 scales) of x per 1x128 group.
    mxfp4: (E4M3 codes, E8M0 bytes) of x per 1x32 block (MXFP8).
    """
    mode = _mode(fp8)
    xs = x if tokens is None else x[np.asarray(tokens)]
    xf = bf16_to_f64(xs)
    if mode == "bf16":
        return xf
    if mode == "fp8":
        return quantize_groups(xf.astype(np.float32))
    return quantize_mx_e4m3(xf.astype(np.float32))


def dispatch(x, p: OraclePlan, fp8):
    """Pool content of the real rows: returns (rows, payload) where ``rows`` are
    pool row indices in ascending order and ``payload`` their values: bf16 bit
    patterns [n, H], or (e4m3 codes [n, H], scales [n, H/128] fp32 | [n, H/32] E8M0)."""
    mode = _mode(fp8)
    rows = np.nonzero(p.src >= 0)[0]
    tok = p.src[rows] // p.K
    if mode == "bf16":
        return rows, bf16_bits(x)[tok]
    codes, scales = token_rows(x, mode)
    return rows, (codes[tok], scales[tok])


# --------------------------------------------------------------------------- #
# A3 + A4: the expert FFN
# --------------------------------------------------------------------------- #
def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):    # exp(-z) = inf for very negative z gives -0
        return z / (1.0 + np.exp(-z))


def expert_weights_f64(w1_e, w1_s_e, w2_e, w2_s_e, dtype=None):
    """One expert's weights, dequantised to float64: (W1 [2I, H], W2 [H, I]).

    ``dtype`` None infers bf16 / fp8 from whether scales are given; "mxfp4" reads
    packed E2M1 codes (uint8 [rows, K/2]) with E8M0 bytes [rows, K/32]."""
    if dtype == "mxfp4":
        return (dequantize_mx_fp4(_np(w1_e), _np(w1_s_e)),
                dequantize_mx_fp4(_np(w2_e), _np(w2_s_e)))
    if w1_s_e is None:
        return bf16_to_f64(w1_e), bf16_to_f64(w2_e)
    return (dequantize_blocks(fp8_codes(w1_e), _np(w1_s_e)),
            dequantize_blocks(fp8_codes(w2_e), _np(w2_s_e)))


def expert_ffn(xrows, W1: np.ndarray, W2: np.ndarray, fp8) -> np.ndarray:
    """y = (silu(X W1_gate^T) * (X W1_up^T)) W2^T for the rows of one expert.

    ``xrows``: float64 [n, H] (bf16), or (codes, scales) of x (fp8, mxfp4). In fp8
    mode h is quantised per 1x128 group from its float32 value before GEMM Y, in
    mxfp4 mode per 1x32 block (MXFP8).
    """
    mode = _mode(fp8)
    if mode == "bf16":
        X = xrows
    elif mode == "fp8":
        X = dequantize_groups(*xrows)
    else:
        X = dequantize_mx_e4m3(*xrows)
    I = W1.shape[0] // 2
    G = X @ W1.T                       # GEMM A: [n, 2I]
    h = silu(G[:, :I]) * G[:, I:]      # gate | up
    if mode == "fp8":
        h = dequantize_groups(*quantize_groups(h.astype(np.float32)))
    elif mode == "mxfp4":
        h = dequantize_mx_e4m3(*quantize_mx_e4m3(h.astype(np.float32)))
    return h @ W2.T                    # GEMM Y: [n, H]


# --------------------------------------------------------------------------- #
# A5: combine
# --------------------------------------------------------------------------- #
def combine(y_pair: np.ndarray, topk_weights, local: np.ndarray) -> np.ndarray:
    """out[t] = sum_k w[t,k] * y_pair[t,k] over local k, in ascending k.

    y_pair: float64 [T, K, H] (rows of non-local pairs are ignored);
    local: bool [T, K]."""
    w = _np(topk_weights).astype(np.float64)
    T, K, H = y_pair.shape
    out = np.zeros((T, H), dtype=np.float64)
    for k in range(K):
        m = local[:, k]
        out[m] += w[m, k][:, None] * y_pair[m, k]
    return out


# --------------------------------------------------------------------------- #
# whole layer
# --------------------------------------------------------------------------- #
@dataclass
class OracleResult:
    plan: OraclePlan
    out: np.ndarray                    # float64 [T or len(tokens), H]
    tokens: Optional[np.ndarray] = None


def moe_layer(inp, tokens: Optional[Sequence[int]] = None, p: Optional[OraclePlan] = None
              ) -> OracleResult:
    """Run the path for all tokens, or only for ``tokens`` (each expert's weights
    are dequantised once, and only for experts those tokens reach)."""
    cfg = inp.cfg
    mode = _mode(cfg.dtype)
    quant = mode != "bf16"
    if p is None:
        p = plan(inp.topk_idx, cfg.expert_begin, cfg.num_local_experts, cfg.tile)
    ids = _np(inp.topk_idx).astype(np.int64)
    T, K = ids.shape
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    sub_ids = ids[toks]
    local = (sub_ids >= cfg.expert_begin) & (sub_ids < cfg.expert_begin + cfg.num_local_experts)
    xin = token_rows(inp.x, mode, toks)
    y_pair = np.zeros((toks.size, K, cfg.H), dtype=np.float64)
    for e in np.unique(sub_ids[local] - cfg.expert_begin):
        W1, W2 = expert_weights_f64(inp.w1[e], None if inp.w1_scale is None else inp.w1_scale[e],
                                    inp.w2[e], None if inp.w2_scale is None else inp.w2_scale[e],
                                    mode if mode == "mxfp4" else None)
        tt, kk = np.nonzero(sub_ids == e + cfg.expert_begin)
        rows = (xin[0][tt], xin[1][tt]) if quant else xin[tt]
        y_pair[tt, kk] = expert_ffn(rows, W1, W2, mode)
    out = combine(y_pair, _np(inp.topk_weights)[toks], local)
    return OracleResult(p, out, None if tokens is None else toks)


def max_norm_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / max|ref| over the whole tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    num = np.abs(got - ref).max()
    return float(num / den) if den > 0 else float(num)
