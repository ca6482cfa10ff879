"""Seeded synthetic inputs for the MoE dispatch -> expert FFN -> combine path.

The layer is the streaming MoE layer of the StreamEP README ("How it works"):
routed (token, k) pairs, per-expert weights ``w1_local`` / ``w2_local`` and
``topk_weights`` go in (README, usage sample). The pages give no data, so every
input here is drawn from a seeded pseudo-random generator with the shapes and
distributions of five workloads:

* ``tiny``        T=64,    H=128,  I=64,   8 experts,            K=2, tile 16, bf16
* ``decode``      T=128,   H=4096, I=1536, 128 experts,          K=8, tile 64, bf16
* ``ep_share``    T=8192,  H=7168, I=2048, 256 experts, 0..31 local, K=8, tile 128, bf16
* ``zipf_skew``   T=16384, H=4096, I=1536, 128 experts, Zipf(1.2) bias, K=8, tile 128, bf16
* ``fp8_weights`` T=8192,  H=4096, I=1536, 128 experts, K=8, tile 128,
  weights e4m3 + fp32 scale per 128x128 block
* ``mxfp4``       T=8192,  H=4096, I=1536, 128 experts, K=8, tile 128,
  weights MXFP4: e2m1 codes + one E8M0 scale per 32 weights along K

Distributions: x ~ N(0,1) rounded to bf16; w1 (gate|up, [2I, H]) and w2
([H, I]) ~ N(0, std 1/sqrt(fan_in)); routing = distinct top-K of per-token
N(0,1) logits (plus log of a Zipf pmf for ``zipf_skew``), topk_weights =
softmax over the K chosen logits.

This module only draws inputs. It holds none of the layer's arithmetic
(placement, GEMMs, activation, quantisation of activations, combine); the CPU
oracle and the GPU path each implement those on their own. It uses torch's CPU
generator (seeded mt19937), so the same values come out on any
host, whatever device later consumes them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

__all__ = [
    "MoEConfig",
    "MoEInputs",
    "CONFIGS",
    "config_by_name",
    "make_x",
    "make_routing",
    "expert_weights",
    "make_inputs",
    "make_dout",
]

# tags keep every stream of draws independent of the others
_TAG_X, _TAG_LOGITS, _TAG_W1, _TAG_W2, _TAG_DOUT = 1, 2, 3, 4, 5


@dataclass(frozen=True)
class MoEConfig:
    """One workload: sizes, routing law and storage dtype."""

    name: str
    T: int                    # tokens
    H: int                    # hidden size
    I: int                    # expert intermediate size (w1 is [2I, H])
    num_experts: int          # experts the router chooses from
    expert_begin: int         # first expert id held by this GPU
    num_local_experts: int    # experts held by this GPU
    K: int                    # top-k
    tile: int                 # pool tile rows
    dtype: str = "bf16"       # "bf16" | "fp8" (weights e4m3 + 128x128 block scales)
                              # | "mxfp4" (weights e2m1 + E8M0 scale per 1x32 along K)
    routing: str = "uniform"  # "uniform" | "zipf1.2"

    @property
    def pairs(self) -> int:
        return self.T * self.K

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS = [
    MoEConfig("tiny", 64, 128, 64, 8, 0, 8, 2, 16, "bf16", "uniform"),
    MoEConfig("decode", 128, 4096, 1536, 128, 0, 128, 8, 64, "bf16", "uniform"),
    MoEConfig("ep_share", 8192, 7168, 2048, 256, 0, 32, 8, 128, "bf16", "uniform"),
    MoEConfig("zipf_skew", 16384, 4096, 1536, 128, 0, 128, 8, 128, "bf16", "zipf1.2"),
    MoEConfig("fp8_weights", 8192, 4096, 1536, 128, 0, 128, 8, 128, "fp8", "uniform"),
    MoEConfig("mxfp4", 8192, 4096, 1536, 128, 0, 128, 8, 128, "mxfp4", "uniform"),
]


def config_by_name(name: str) -> MoEConfig:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def _seed(base: int, tag: int, index: int = 0) -> int:
    # a fixed injective mix of (base, tag, index) into a 63-bit torch seed
    return ((base * 1_000_003 + tag) * 1_000_033 + index) & 0x7FFF_FFFF_FFFF_FFFF


def _gen(base: int, tag: int, index: int = 0) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(_seed(base, tag, index))


def base_seed(cfg: MoEConfig, seed: Optional[int] = None) -> int:
    """Default seed of a workload: 1000 + its index in CONFIGS (or a hash of its name)."""
    if seed is not None:
        return int(seed)
    for i, c in enumerate(CONFIGS):
        if c == cfg:
            return 1000 + i
    return 1000 + (sum(map(ord, cfg.name)) * 131 + cfg.T * 7 + cfg.H) % 100_000


def make_x(cfg: MoEConfig, seed: int) -> torch.Tensor:
    """x[T, H] ~ N(0, 1), rounded to bf16 (round-to-nearest-even)."""
    return torch.randn(cfg.T, cfg.H, generator=_gen(seed, _TAG_X)).to(torch.bfloat16)


def make_dout(cfg: MoEConfig, seed: int) -> torch.Tensor:
    """The layer's output gradient dout[T, H] ~ N(0, 1), rounded to bf16 (backward pass input)."""
    return torch.randn(cfg.T, cfg.H, generator=_gen(seed, _TAG_DOUT)).to(torch.bfloat16)


def make_routing(cfg: MoEConfig, seed: int):
    """Distinct top-K of per-token logits and softmax weights over the K chosen.

    Returns (topk_idx int32 [T, K] with global expert ids, topk_weights float32 [T, K]).
    k = 0 is the largest logit; equal logits go to the lower expert id.
    ``zipf1.2`` adds log p_e with p_e proportional to (e+1)^-1.2 to every token's logits,
    so expert 0 is the most popular and the tail experts can go empty.
    """
    E = cfg.num_experts
    logits = torch.randn(cfg.T, E, generator=_gen(seed, _TAG_LOGITS)).numpy()
    if cfg.routing == "zipf1.2":
        p = (np.arange(1, E + 1, dtype=np.float64)) ** -1.2
        p /= p.sum()
        logits = (logits.astype(np.float64) + np.log(p)[None, :]).astype(np.float32)
    elif cfg.routing != "uniform":
        raise ValueError(f"unknown routing {cfg.routing!r}")
    order = np.argsort(-logits, axis=1, kind="stable")[:, : cfg.K]
    chosen = np.take_along_axis(logits, order, axis=1).astype(np.float32)
    z = np.exp(chosen - chosen.max(axis=1, keepdims=True), dtype=np.float32)
    w = (z / z.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return (torch.from_numpy(np.ascontiguousarray(order.astype(np.int32))),
            torch.from_numpy(np.ascontiguousarray(w)))


def _block_quant_e4m3(w: torch.Tensor):
    """Block-quantise an fp32 master [R, C] to e4m3 codes with one fp32 scale per 128x128 block.

    scale = amax(block) / 448 (1 if the block is all zero); codes = e4m3(w / scale)
    through torch's own cast, after clamping to the finite range. This is how the
    fp8 workload's stored weights are defined; the layer only reads them.
    """
    R, C = w.shape
    assert R % 128 == 0 and C % 128 == 0, (R, C)
    blocks = w.reshape(R // 128, 128, C // 128, 128)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    q = (blocks / scale[:, None, :, None]).clamp_(-448.0, 448.0).reshape(R, C)
    return q.to(torch.float8_e4m3fn), scale.contiguous()


# e2m1 magnitudes by code (OCP MX e2m1: 1 sign, 2 exponent bits with bias 1, 1 mantissa bit)
_E2M1_GRID = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MIDS = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / 2


def _mx_quant_e2m1(w: torch.Tensor):
    """MXFP4-quantise an fp32 master [R, C] along C in blocks of 32.

    Per block: shared exponent = floor(log2(amax)) - 2 (the largest e2m1 power,
    6 = 1.5 * 2^2), clamped to [-127, 127]; E8M0 byte = exponent + 127 (0 for an
    all-zero block). Codes = e2m1 of w / 2^exponent, round to nearest, ties to the
    even code, magnitudes above 6 saturate to 6. Two codes per byte, the even
    column in the low nibble. This is how the workload's stored weights are
    defined; the layer only reads them.
    """
    R, C = w.shape
    assert C % 32 == 0, C
    blk = w.reshape(R, C // 32, 32)
    amax = blk.abs().amax(dim=2)
    _, ex = torch.frexp(amax)                       # amax = m * 2^ex, m in [0.5, 1)
    shared = torch.where(amax > 0, ex - 1 - 2, torch.full_like(ex, -127)).clamp_(-127, 127)
    v = blk / torch.ldexp(torch.ones_like(amax), shared)[..., None]
    a = v.abs().clamp_(max=6.0)
    # nearest grid point: count the midpoints below (lo) and at-or-below (hi);
    # they differ only on an exact midpoint, where the even code wins
    lo = torch.bucketize(a, _E2M1_MIDS, right=False)
    hi = torch.bucketize(a, _E2M1_MIDS, right=True)
    code = torch.where((lo == hi) | (lo % 2 == 0), lo, hi)
    code = code | torch.where(v < 0, 8, 0)
    code = code.reshape(R, C).to(torch.uint8)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    return packed, (shared + 127).to(torch.uint8).contiguous()


def expert_weights(cfg: MoEConfig, seed: int, e_local: int):
    """Weights of local expert ``e_local``: (w1 [2I, H], w1_scale, w2 [H, I], w2_scale).

    Scales are None for bf16 storage. Each expert has its own generators, so any
    subset of experts can be drawn alone and matches the full draw.
    """
    H, I = cfg.H, cfg.I
    e_glob = cfg.expert_begin + e_local
    w1 = torch.randn(2 * I, H, generator=_gen(seed, _TAG_W1, e_glob)) * (1.0 / math.sqrt(H))
    w2 = torch.randn(H, I, generator=_gen(seed, _TAG_W2, e_glob)) * (1.0 / math.sqrt(I))
    if cfg.dtype == "bf16":
        return w1.to(torch.bfloat16), None, w2.to(torch.bfloat16), None
    if cfg.dtype == "fp8":
        q1, s1 = _block_quant_e4m3(w1)
        q2, s2 = _block_quant_e4m3(w2)
        return q1, s1, q2, s2
    if cfg.dtype == "mxfp4":
        q1, s1 = _mx_quant_e2m1(w1)
        q2, s2 = _mx_quant_e2m1(w2)
        return q1, s1, q2, s2
    raise ValueError(cfg.dtype)


@dataclass
class MoEInputs:
    cfg: MoEConfig
    seed: int
    x: torch.Tensor                   # bf16 [T, H]
    topk_idx: torch.Tensor            # int32 [T, K], global expert ids
    topk_weights: torch.Tensor        # float32 [T, K]
    w1: Optional[torch.Tensor]        # bf16 | float8_e4m3fn [E_local, 2I, H] | uint8 [E_local, 2I, H/2] (mxfp4)
    w1_scale: Optional[torch.Tensor]  # float32 [E_local, 2I/128, H/128] (fp8) | uint8 [E_local, 2I, H/32] (mxfp4)
    w2: Optional[torch.Tensor]        # bf16 | float8_e4m3fn [E_local, H, I] | uint8 [E_local, H, I/2] (mxfp4)
    w2_scale: Optional[torch.Tensor]  # float32 [E_local, H/128, I/128] (fp8) | uint8 [E_local, H, I/32] (mxfp4)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(cfg: MoEConfig, seed: Optional[int] = None, *, weights: bool = True,
                pin_memory: bool = False) -> MoEInputs:
    """Draw every input of one workload on the host (CPU tensors).

    With ``pin_memory`` the big tensors land in page-locked host memory so that
    the upload to the GPU is a plain DMA.
    """
    s = base_seed(cfg, seed)
    x = make_x(cfg, s)
    idx, w = make_routing(cfg, s)
    if pin_memory:
        x = x.pin_memory()
    if not weights:
        return MoEInputs(cfg, s, x, idx, w, None, None, None, None)
    E, H, I = cfg.num_local_experts, cfg.H, cfg.I
    mx = cfg.dtype == "mxfp4"
    fp8 = cfg.dtype == "fp8"
    if mx:
        w1 = torch.empty(E, 2 * I, H // 2, dtype=torch.uint8, pin_memory=pin_memory)
        w2 = torch.empty(E, H, I // 2, dtype=torch.uint8, pin_memory=pin_memory)
        w1s = torch.empty(E, 2 * I, H // 32, dtype=torch.uint8)
        w2s = torch.empty(E, H, I // 32, dtype=torch.uint8)
    else:
        wdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float8_e4m3fn
        w1 = torch.empty(E, 2 * I, H, dtype=wdt, pin_memory=pin_memory)
        w2 = torch.empty(E, H, I, dtype=wdt, pin_memory=pin_memory)
        w1s = torch.empty(E, 2 * I // 128, H // 128, dtype=torch.float32) if fp8 else None
        w2s = torch.empty(E, H // 128, I // 128, dtype=torch.float32) if fp8 else None

    def one(e):
        a, as_, b, bs = expert_weights(cfg, s, e)
        w1[e].copy_(a)
        w2[e].copy_(b)
        if fp8 or mx:
            w1s[e].copy_(as_)
            w2s[e].copy_(bs)

    if E == 1:
        one(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(E)))
    return MoEInputs(cfg, s, x, idx, w, w1, w1s, w2, w2s)
