"""Python binding of libmoe355: the MoE dispatch -> expert FFN -> combine path.

Argument marshalling only: every step runs in the library's HIP kernels.
torch supplies device memory and streams. The entry points keep the C ABI's
names (include/moe355.h); ``StreamMoE`` / ``stream_moe`` string them together
the way the StreamEP README's usage sample calls ``stream_moe_func``
(x, topk_idx, topk_weights, w1_local, w2_local, streams).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _abi
from ._abi import (MOE_BF16, MOE_FP8_E4M3_G128, MOE_MXFP4, MOE_WEIGHTS_MFMA_TILED, MOE_WEIGHTS_ROW_MAJOR,
                   MoeError, PlanT, TileConfig, check, load)

__all__ = [
    "MOE_BF16", "MOE_FP8_E4M3_G128", "MOE_MXFP4", "MoeError", "Plan", "Workspace", "TileConfig",
    "pool_rows_upper_bound", "workspace_bytes", "moe_plan", "moe_plan_noalloc", "moe_query_pool_rows",
    "moe_dispatch", "moe_expert_ffn", "moe_expert_ffn_combine", "moe_combine", "moe_get_error",
    "moe_pack_weights",
    "moe_pack_mx_scales", "moe_expert_ffn_train", "moe_combine_backward", "moe_expert_ffn_backward",
    "moe_dispatch_backward", "moe_pack_weights_transposed",
    "device_cu_count", "MOE_WEIGHTS_ROW_MAJOR", "MOE_WEIGHTS_MFMA_TILED",
    "make_streams", "StreamMoE", "stream_moe",
]


def _vp(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(s) -> ctypes.c_void_p:
    if s is None:
        s = torch.cuda.current_stream()
    if isinstance(s, torch.cuda.Stream):
        return ctypes.c_void_p(s.cuda_stream)
    return ctypes.c_void_p(int(s))


def _dtype_code(dtype) -> int:
    if dtype in ("bf16", MOE_BF16):
        return MOE_BF16
    if dtype in ("fp8", MOE_FP8_E4M3_G128):
        return MOE_FP8_E4M3_G128
    if dtype in ("mxfp4", MOE_MXFP4):
        return MOE_MXFP4
    raise ValueError(f"dtype {dtype!r}")


_DTYPE_NAMES = {MOE_BF16: "bf16", MOE_FP8_E4M3_G128: "fp8", MOE_MXFP4: "mxfp4"}


def _need_cuda(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def pool_rows_upper_bound(T: int, K: int, E_local: int, tile: int) -> int:
    return int(load().moe_pool_rows_upper_bound(T, K, E_local, tile))


def workspace_bytes(T: int, K: int, E_local: int, tile: int, pool_rows: int = 0, I: int = 0,
                    dtype="bf16") -> int:
    return int(load().moe_workspace_bytes(T, K, E_local, tile, pool_rows, I, _dtype_code(dtype)))


def device_cu_count() -> int:
    return int(load().moe_device_cu_count())


@dataclass
class Plan:
    """Caller-owned plan arrays (moe_plan_t) on one device."""

    T: int
    K: int
    expert_begin: int
    E_local: int
    tile: int
    rows_cap: int
    counts: torch.Tensor
    offsets: torch.Tensor
    pos: torch.Tensor
    src: torch.Tensor
    tile_expert: torch.Tensor
    num_tiles: torch.Tensor
    tile_ready: torch.Tensor

    @classmethod
    def allocate(cls, T, K, expert_begin, E_local, tile, device="cuda") -> "Plan":
        cap = pool_rows_upper_bound(T, K, E_local, tile)
        if cap == 0:
            raise MoeError("moe_pool_rows_upper_bound", _abi.MOE_ERR_INVALID)
        i32 = dict(dtype=torch.int32, device=device)
        return cls(T, K, expert_begin, E_local, tile, cap,
                   torch.empty(E_local, **i32), torch.empty(E_local + 1, **i32),
                   torch.empty(T * K, **i32), torch.empty(cap, **i32),
                   torch.empty(cap // tile, **i32), torch.empty(1, **i32),
                   torch.zeros(cap // tile, dtype=torch.int32, device=device))

    def c(self) -> PlanT:
        return PlanT(self.T, self.K, self.expert_begin, self.E_local, self.tile, self.rows_cap,
                     self.counts.data_ptr(), self.offsets.data_ptr(), self.pos.data_ptr(),
                     self.src.data_ptr(), self.tile_expert.data_ptr(), self.num_tiles.data_ptr(),
                     self.tile_ready.data_ptr())


class Workspace:
    """Zero-initialised device workspace shared by plan, dispatch, FFN and error queries."""

    def __init__(self, T, K, E_local, tile, pool_rows=0, I=0, dtype="bf16", device="cuda"):
        n = workspace_bytes(T, K, E_local, tile, pool_rows, I, dtype)
        if n == 0:
            raise MoeError("moe_workspace_bytes", _abi.MOE_ERR_INVALID)
        self.buf = torch.zeros(n, dtype=torch.uint8, device=device)

    @property
    def nbytes(self) -> int:
        return self.buf.numel()


def moe_plan(topk_idx: torch.Tensor, plan: Plan, ws: Workspace, stream=None) -> None:
    _need_cuda(topk_idx, "topk_idx", torch.int32)
    if topk_idx.shape != (plan.T, plan.K):
        raise ValueError(f"topk_idx shape {tuple(topk_idx.shape)} != {(plan.T, plan.K)}")
    c = plan.c()
    check("moe_plan", load().moe_plan(_vp(topk_idx), ctypes.byref(c), _vp(ws.buf), ws.nbytes,
                                      _stream(stream)))


def moe_plan_noalloc(topk_idx: torch.Tensor, plan: Plan, stream=None) -> None:
    """moe_plan with the library's own device scratch instead of a workspace (nothing is
    allocated; calls that overlap on one device race)."""
    _need_cuda(topk_idx, "topk_idx", torch.int32)
    if topk_idx.shape != (plan.T, plan.K):
        raise ValueError(f"topk_idx shape {tuple(topk_idx.shape)} != {(plan.T, plan.K)}")
    c = plan.c()
    check("moe_plan_noalloc", load().moe_plan_noalloc(_vp(topk_idx), ctypes.byref(c), _stream(stream)))


def moe_query_pool_rows(plan: Plan, stream=None) -> int:
    out = ctypes.c_int32(0)
    c = plan.c()
    check("moe_query_pool_rows", load().moe_query_pool_rows(ctypes.byref(c), ctypes.byref(out),
                                                            _stream(stream)))
    return int(out.value)


def moe_dispatch(x: torch.Tensor, plan: Plan, pool: torch.Tensor, pool_s: Optional[torch.Tensor],
                 epoch: int, ws: Workspace, dtype="bf16", stream=None) -> None:
    _need_cuda(x, "x", torch.bfloat16)
    _need_cuda(pool, "pool")
    if x.shape[0] != plan.T:
        raise ValueError("x rows != T")
    code = _dtype_code(dtype)
    H = x.shape[1]
    rows = pool.shape[0]
    c = plan.c()
    check("moe_dispatch", load().moe_dispatch(_vp(x), H, code, ctypes.byref(c), rows, _vp(pool),
                                              _vp(pool_s), epoch, _vp(ws.buf), ws.nbytes,
                                              _stream(stream)))


def _ffn_shapes(plan: Plan, pool, w1, w2, y_pool, code):
    for t, n in ((pool, "pool"), (w1, "w1"), (w2, "w2"), (y_pool, "y_pool")):
        _need_cuda(t, n)
    E, twoI, H = w1.shape
    if code == MOE_MXFP4:          # packed e2m1: two codes per byte along K
        H *= 2
        if E != plan.E_local or w2.shape != (E, H, twoI // 4):
            raise ValueError("mxfp4 w1 [E_local, 2I, H/2] / w2 [E_local, H, I/2] shapes do not match")
    elif E != plan.E_local or w2.shape != (E, H, twoI // 2):
        raise ValueError("w1 [E_local, 2I, H] / w2 [E_local, H, I] shapes do not match")
    if y_pool.shape[0] != pool.shape[0] or y_pool.shape[1] != H:
        raise ValueError("y_pool must be [pool rows, H]")
    return H, twoI // 2


def moe_expert_ffn(plan: Plan, pool: torch.Tensor, pool_s: Optional[torch.Tensor],
                   w1: torch.Tensor, w1_s: Optional[torch.Tensor], w2: torch.Tensor,
                   w2_s: Optional[torch.Tensor], epoch: int, ws: Workspace, y_pool: torch.Tensor,
                   dtype="bf16", cfg: Optional[TileConfig] = None, stream=None) -> None:
    code = _dtype_code(dtype)
    H, I = _ffn_shapes(plan, pool, w1, w2, y_pool, code)
    c = plan.c()
    cfgp = ctypes.byref(cfg) if cfg is not None else None
    check("moe_expert_ffn", load().moe_expert_ffn(
        ctypes.byref(c), pool.shape[0], _vp(pool), _vp(pool_s), _vp(w1), _vp(w1_s), _vp(w2),
        _vp(w2_s), H, I, code, epoch, _vp(ws.buf), ws.nbytes, _vp(y_pool),
        cfgp, _stream(stream)))


def moe_expert_ffn_combine(plan: Plan, pool: torch.Tensor, pool_s: Optional[torch.Tensor],
                           w1: torch.Tensor, w1_s: Optional[torch.Tensor], w2: torch.Tensor,
                           w2_s: Optional[torch.Tensor], epoch: int, ws: Workspace, y_pool: torch.Tensor,
                           topk_weights: torch.Tensor, out: torch.Tensor, dtype="bf16",
                           cfg: Optional[TileConfig] = None, stream=None) -> None:
    """moe_expert_ffn then moe_combine, with combine on completion inside GEMM Y."""
    code = _dtype_code(dtype)
    H, I = _ffn_shapes(plan, pool, w1, w2, y_pool, code)
    _need_cuda(topk_weights, "topk_weights", torch.float32)
    _need_cuda(out, "out", torch.bfloat16)
    if topk_weights.shape != (plan.T, plan.K) or out.shape != (plan.T, H):
        raise ValueError("topk_weights [T, K] / out [T, H] shapes do not match the plan")
    c = plan.c()
    cfgp = ctypes.byref(cfg) if cfg is not None else None
    check("moe_expert_ffn_combine", load().moe_expert_ffn_combine(
        ctypes.byref(c), pool.shape[0], _vp(pool), _vp(pool_s), _vp(w1), _vp(w1_s), _vp(w2),
        _vp(w2_s), H, I, code, epoch, _vp(ws.buf), ws.nbytes, _vp(y_pool), _vp(topk_weights), _vp(out),
        cfgp, _stream(stream)))


def moe_expert_ffn_train(plan: Plan, pool: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, epoch: int,
                         ws: Workspace, y_pool: torch.Tensor, g_pool: torch.Tensor,
                         cfg: Optional[TileConfig] = None, stream=None) -> None:
    """Training forward (bf16): moe_expert_ffn that also keeps G = [gate | up] in g_pool."""
    H, I = _ffn_shapes(plan, pool, w1, w2, y_pool, MOE_BF16)
    _need_cuda(g_pool, "g_pool", torch.bfloat16)
    if g_pool.shape != (pool.shape[0], 2 * I):
        raise ValueError("g_pool must be [pool rows, 2I]")
    c = plan.c()
    cfgp = ctypes.byref(cfg) if cfg is not None else None
    check("moe_expert_ffn_train", load().moe_expert_ffn_train(
        ctypes.byref(c), pool.shape[0], _vp(pool), _vp(w1), _vp(w2), H, I, epoch, _vp(ws.buf), ws.nbytes,
        _vp(y_pool), _vp(g_pool), cfgp, _stream(stream)))


def moe_combine_backward(dout: torch.Tensor, topk_weights: torch.Tensor, y_pool: torch.Tensor, plan: Plan,
                         dy_pool: torch.Tensor, d_topk_weights: torch.Tensor, epoch: int, ws: Workspace,
                         stream=None) -> None:
    """dy_pool[pos[t,k]] = w[t,k] dout[t]; d_topk_weights[t,k] = <dout[t], y_pool[pos[t,k]]>.
    dy_pool may be y_pool itself (each row is read before it is overwritten, by the same lane).
    Raises each pool tile's ready flag to ``epoch`` once its dy rows are stored."""
    _need_cuda(dout, "dout", torch.bfloat16)
    _need_cuda(topk_weights, "topk_weights", torch.float32)
    _need_cuda(d_topk_weights, "d_topk_weights", torch.float32)
    _need_cuda(y_pool, "y_pool", torch.bfloat16)
    _need_cuda(dy_pool, "dy_pool", torch.bfloat16)
    if dout.shape[0] != plan.T or topk_weights.shape != (plan.T, plan.K) or d_topk_weights.shape != (plan.T, plan.K):
        raise ValueError("dout [T, H] / topk_weights / d_topk_weights [T, K] do not match the plan")
    if dy_pool.shape != y_pool.shape or y_pool.shape[1] != dout.shape[1]:
        raise ValueError("dy_pool and y_pool must be [pool rows, H]")
    c = plan.c()
    check("moe_combine_backward", load().moe_combine_backward(
        _vp(dout), _vp(topk_weights), _vp(y_pool), y_pool.shape[0], ctypes.byref(c), dout.shape[1], _vp(dy_pool),
        _vp(d_topk_weights), epoch, _vp(ws.buf), ws.nbytes, _stream(stream)))


def moe_expert_ffn_backward(plan: Plan, pool: torch.Tensor, dy_pool: torch.Tensor, g_pool: torch.Tensor,
                            w1t: torch.Tensor, w2t: torch.Tensor, epoch: int, ws: Workspace, dx_pool: torch.Tensor,
                            dw1: torch.Tensor, dw2: torch.Tensor, cfg: Optional[TileConfig] = None,
                            stream=None) -> None:
    """Backward grouped GEMMs Y and A; g_pool's G is replaced by dG. Backward Y's units wait
    for the ready flags moe_combine_backward raised with the same ``epoch``."""
    for t, n in ((pool, "pool"), (dy_pool, "dy_pool"), (g_pool, "g_pool"), (w1t, "w1t"), (w2t, "w2t"),
                 (dx_pool, "dx_pool"), (dw1, "dw1"), (dw2, "dw2")):
        _need_cuda(t, n, torch.bfloat16)
    rows, H = pool.shape
    E, Ht, twoI = w1t.shape
    I = twoI // 2
    if Ht != H or E != plan.E_local or w2t.shape != (E, I, H) or g_pool.shape != (rows, twoI):
        raise ValueError("w1t [E_local, H, 2I] / w2t [E_local, I, H] / g_pool [rows, 2I] do not match")
    if dy_pool.shape != (rows, H) or dx_pool.shape != (rows, H):
        raise ValueError("dy_pool / dx_pool must be [pool rows, H]")
    if dw1.shape != (E, twoI, H) or dw2.shape != (E, H, I):
        raise ValueError("dw1 [E_local, 2I, H] / dw2 [E_local, H, I] do not match")
    c = plan.c()
    cfgp = ctypes.byref(cfg) if cfg is not None else None
    check("moe_expert_ffn_backward", load().moe_expert_ffn_backward(
        ctypes.byref(c), rows, _vp(pool), _vp(dy_pool), _vp(g_pool), _vp(w1t), _vp(w2t), H, I, epoch,
        _vp(ws.buf), ws.nbytes, _vp(dx_pool), _vp(dw1), _vp(dw2), cfgp, _stream(stream)))


def moe_dispatch_backward(dx_pool: torch.Tensor, plan: Plan, dx: torch.Tensor, stream=None) -> None:
    """dx[t] = sum over the token's local pairs of dx_pool[pos[t,k]]."""
    _need_cuda(dx_pool, "dx_pool", torch.bfloat16)
    _need_cuda(dx, "dx", torch.bfloat16)
    if dx.shape[0] != plan.T or dx.shape[1] != dx_pool.shape[1]:
        raise ValueError("dx must be [T, H]")
    c = plan.c()
    check("moe_dispatch_backward", load().moe_dispatch_backward(
        _vp(dx_pool), dx_pool.shape[0], ctypes.byref(c), dx.shape[1], _vp(dx), _stream(stream)))


def moe_pack_weights_transposed(w: torch.Tensor, dtype="bf16", stream=None) -> torch.Tensor:
    """w [E, rows, K] (bf16) -> the tiled layout of each w[e]^T, a new [E, K, rows] tensor."""
    _need_cuda(w, "w")
    E, rows, K = w.shape
    out = torch.empty(E, K, rows, dtype=w.dtype, device=w.device)
    check("moe_pack_weights_transposed", load().moe_pack_weights_transposed(
        _vp(w), E, rows, K, _dtype_code(dtype), _vp(out), _stream(stream)))
    return out


def moe_combine(y_pool: torch.Tensor, topk_weights: torch.Tensor, plan: Plan, out: torch.Tensor,
                stream=None) -> None:
    _need_cuda(y_pool, "y_pool")
    _need_cuda(topk_weights, "topk_weights", torch.float32)
    _need_cuda(out, "out", torch.bfloat16)
    if topk_weights.shape != (plan.T, plan.K) or out.shape[0] != plan.T:
        raise ValueError("topk_weights [T, K] / out [T, H] shapes do not match the plan")
    c = plan.c()
    check("moe_combine", load().moe_combine(_vp(y_pool), y_pool.shape[0], _vp(topk_weights),
                                            ctypes.byref(c), out.shape[1], _vp(out), _stream(stream)))


def moe_pack_weights(w: torch.Tensor, dtype="bf16", stream=None) -> torch.Tensor:
    """Permute expert weights [E, rows, K] (mxfp4: packed codes [E, rows, K/2]) into MFMA
    fragment order (a new tensor)."""
    _need_cuda(w, "w")
    E, rows, K = w.shape
    if _dtype_code(dtype) == MOE_MXFP4:
        K *= 2
    out = torch.empty_like(w)
    check("moe_pack_weights", load().moe_pack_weights(_vp(w), E, rows, K, _dtype_code(dtype), _vp(out),
                                                      _stream(stream)))
    return out


def moe_pack_mx_scales(s: torch.Tensor, stream=None) -> torch.Tensor:
    """Permute MXFP4 weight scales [E, rows, K/32] (E8M0 bytes) into the scaled MFMA's
    operand order (a new tensor)."""
    _need_cuda(s, "s", torch.uint8)
    E, rows, kb = s.shape
    out = torch.empty_like(s)
    check("moe_pack_mx_scales", load().moe_pack_mx_scales(_vp(s), E, rows, kb * 32, _vp(out), _stream(stream)))
    return out


def moe_get_error(ws: Workspace, stream=None) -> int:
    return int(load().moe_get_error(_vp(ws.buf), ws.nbytes, _stream(stream)))


def make_streams(device=None) -> Tuple[torch.cuda.Stream, torch.cuda.Stream]:
    """(compute, comm) streams at the default priority."""
    return torch.cuda.Stream(device=device), torch.cuda.Stream(device=device)


class StreamMoE:
    """Buffers of one layer shape, and the four calls in order.

    The pool, h and y_pool are sized by the sync-free bound
    (``pool_rows_upper_bound``) unless ``pool_rows`` is given.
    """

    def __init__(self, T, H, I, K, num_local_experts, *, expert_begin=0, tile=128, dtype="bf16",
                 device="cuda", pool_rows: Optional[int] = None, cfg: Optional[TileConfig] = None,
                 weight_layout: str = "auto", combine_on_completion: bool = False, train: bool = False):
        self.T, self.H, self.I, self.K = T, H, I, K
        # GEMM Y's workgroups combine each token once its tiles are done (no FFN -> combine join)
        self.combine_on_completion = combine_on_completion
        self.E_local, self.expert_begin, self.tile = num_local_experts, expert_begin, tile
        self.dtype = _DTYPE_NAMES[_dtype_code(dtype)]
        # tiled weights feed the big-tile kernel, which needs whole 512-column blocks
        # (bf16: tile 64 or 128; fp8, mxfp4: tile 128); mxfp4 runs there only
        tiles_ok = tile in (64, 128) if self.dtype == "bf16" else tile == 128
        block_ok = cfg is None or cfg.block_n in (0, 512)
        tiled_ok = tiles_ok and I % 256 == 0 and H % 512 == 0 and block_ok
        # the 256 x 256 units take tiled bf16 weights at tile 128 for H % 256, I % 128
        if (self.dtype == "bf16" and tile == 128 and H % 256 == 0 and I % 128 == 0 and block_ok
                and not combine_on_completion and (cfg is None or cfg.unit_rows != 128)):
            tiled_ok = True
        if (weight_layout == "tiled" or self.dtype == "mxfp4") and not tiled_ok:
            raise MoeError("StreamMoE", _abi.MOE_ERR_UNSUPPORTED)
        if self.dtype == "mxfp4" and weight_layout == "row_major":
            raise MoeError("StreamMoE", _abi.MOE_ERR_UNSUPPORTED)
        self.tiled = weight_layout == "tiled" or (weight_layout == "auto" and tiled_ok)
        if cfg is None:
            cfg = TileConfig(0, 0, 0, 0, 0, 0, 0)
        cfg.weight_layout = MOE_WEIGHTS_MFMA_TILED if self.tiled else MOE_WEIGHTS_ROW_MAJOR
        self.cfg = cfg
        self.plan = Plan.allocate(T, K, expert_begin, num_local_experts, tile, device)
        rows = pool_rows or self.plan.rows_cap
        self.pool_rows = rows
        self.ws = Workspace(T, K, num_local_experts, tile, rows, I, self.dtype, device)
        if self.dtype == "bf16":
            self.pool = torch.empty(rows, H, dtype=torch.bfloat16, device=device)
            self.pool_s = None
        elif self.dtype == "fp8":
            self.pool = torch.empty(rows, H, dtype=torch.uint8, device=device)
            self.pool_s = torch.empty(rows, H // 128, dtype=torch.float32, device=device)   # tile-major words
        else:
            self.pool = torch.empty(rows, H, dtype=torch.uint8, device=device)
            self.pool_s = torch.empty(rows, (H + 127) // 128 * 4, dtype=torch.uint8, device=device)
        self.y_pool = torch.empty(rows, H, dtype=torch.bfloat16, device=device)
        self.out = torch.empty(T, H, dtype=torch.bfloat16, device=device)
        self.epoch = 0
        # training: G kept by the forward (replaced by dG in backward), and the backward's buffers
        self.train = train
        if train:
            if self.dtype != "bf16" or not self.tiled:
                raise MoeError("StreamMoE(train=True)", _abi.MOE_ERR_UNSUPPORTED)
            self.g_pool = torch.empty(rows, 2 * I, dtype=torch.bfloat16, device=device)
            self.dx_pool = torch.empty(rows, H, dtype=torch.bfloat16, device=device)
            self.dx = torch.empty(T, H, dtype=torch.bfloat16, device=device)
            self.dw = torch.empty(T, K, dtype=torch.float32, device=device)

    def prepare_weights(self, w1, w2, w1_scale=None, w2_scale=None):
        """(w1, w2, w1_scale, w2_scale) as forward() wants them: permuted once into MFMA fragment
        order when the layer uses tiled weights (a load-time step, like any weight
        preprocessing), MXFP4 scales into operand order, else as is."""
        if not self.tiled:
            return w1, w2, w1_scale, w2_scale
        if self.dtype == "mxfp4":
            w1_scale, w2_scale = moe_pack_mx_scales(w1_scale), moe_pack_mx_scales(w2_scale)
        return moe_pack_weights(w1, self.dtype), moe_pack_weights(w2, self.dtype), w1_scale, w2_scale

    def prepare_backward_weights(self, w1, w2):
        """(w1t, w2t): the transposed, tiled weights the backward data GEMMs read (load time)."""
        return moe_pack_weights_transposed(w1), moe_pack_weights_transposed(w2)

    def backward(self, dout, topk_weights, w1t, w2t, streams=None):
        """Gradients of the last forward (train=True) for the output gradient dout [T, H]:
        returns (dx [T, H] bf16, d_topk_weights [T, K] fp32, dw1 [E_local, 2I, H], dw2 [E_local, H, I]).
        y_pool is overwritten by dy. ``streams=(compute, comm)`` mirrors forward(): combine
        backward on comm raises each pool tile's flag as its dy rows land, and the backward GEMMs
        on compute start on flagged tiles (backward Y's grid leaves CUs for combine backward);
        dispatch backward follows on comm. None runs everything on the current stream."""
        if not self.train:
            raise RuntimeError("StreamMoE was built without train=True")
        epoch = self.next_epoch()
        dw1 = torch.empty(self.E_local, 2 * self.I, self.H, dtype=torch.bfloat16, device=dout.device)
        dw2 = torch.empty(self.E_local, self.H, self.I, dtype=torch.bfloat16, device=dout.device)
        if streams is None:
            s = torch.cuda.current_stream()
            moe_combine_backward(dout, topk_weights, self.y_pool, self.plan, self.y_pool, self.dw, epoch, self.ws, s)
            moe_expert_ffn_backward(self.plan, self.pool, self.y_pool, self.g_pool, w1t, w2t, epoch, self.ws,
                                    self.dx_pool, dw1, dw2, self.cfg, s)
            moe_dispatch_backward(self.dx_pool, self.plan, self.dx, s)
            return self.dx, self.dw, dw1, dw2
        compute, comm = streams
        cur = torch.cuda.current_stream()
        comm.wait_stream(cur)
        compute.wait_stream(cur)            # w1t / w2t and the new dw1 / dw2 belong to the caller's stream
        moe_combine_backward(dout, topk_weights, self.y_pool, self.plan, self.y_pool, self.dw, epoch, self.ws, comm)
        moe_expert_ffn_backward(self.plan, self.pool, self.y_pool, self.g_pool, w1t, w2t, epoch, self.ws,
                                self.dx_pool, dw1, dw2, self._concurrent_cfg(), compute)
        done = torch.cuda.Event()
        done.record(compute)
        comm.wait_event(done)
        moe_dispatch_backward(self.dx_pool, self.plan, self.dx, comm)
        cur.wait_stream(comm)
        return self.dx, self.dw, dw1, dw2

    def check_errors(self, stream=None) -> None:
        """Wait for ``stream`` and raise MoeError if the device recorded an error since the last
        check (a ready-flag wait that timed out, a pool too small for the plan). forward() is
        asynchronous and does not synchronise, so device errors surface only here (or through
        moe_get_error); the error word is cleared by reading it."""
        rc = moe_get_error(self.ws, stream)
        if rc != 0:
            raise MoeError("device", rc)

    def _concurrent_cfg(self) -> TileConfig:
        """The tile config of an FFN that runs while dispatch may still be running on another
        stream: GEMM A's persistent grid leaves CUs free for dispatch (one GEMM workgroup fills a
        CU), so that GEMM A's waits for tiles always end. One eighth of the CUs unless the
        caller's config sets dispatch_cus."""
        c = self.cfg
        if c.dispatch_cus > 0:
            return c
        if getattr(self, "_ccfg", None) is None:
            self._ccfg = TileConfig(c.block_n, c.gemm_workgroups, c.spin_timeout_us, c.unit_order,
                                    c.weight_layout, c.a_stages, max(1, device_cu_count() // 8))
        return self._ccfg

    def next_epoch(self) -> int:
        self.epoch = (self.epoch % 0xFFFFFFFF) + 1      # 1 .. 2^32-1; 0 is never a valid epoch
        return self.epoch

    def forward(self, x, topk_idx, topk_weights, w1, w2, w1_scale=None, w2_scale=None,
                streams=None) -> torch.Tensor:
        """One layer. Weights and scales come from prepare_weights(). ``streams=(compute, comm)`` runs
        plan/dispatch/combine on comm and the FFN on compute, ordered by events, with GEMM A
        claiming pool tiles as dispatch raises their flags (its grid then leaves CUs free for
        dispatch); None runs everything on the current stream. Asynchronous: device errors are
        reported by check_errors()."""
        if topk_idx.dtype != torch.int32:
            topk_idx = topk_idx.to(torch.int32)
        epoch = self.next_epoch()
        if streams is None:
            s = torch.cuda.current_stream()
            moe_plan(topk_idx, self.plan, self.ws, s)
            moe_dispatch(x, self.plan, self.pool, self.pool_s, epoch, self.ws, self.dtype, s)
            if self.combine_on_completion:
                moe_expert_ffn_combine(self.plan, self.pool, self.pool_s, w1, w1_scale, w2, w2_scale, epoch,
                                       self.ws, self.y_pool, topk_weights, self.out, self.dtype, self.cfg, s)
                return self.out
            if self.train:
                moe_expert_ffn_train(self.plan, self.pool, w1, w2, epoch, self.ws, self.y_pool, self.g_pool,
                                     self.cfg, s)
            else:
                moe_expert_ffn(self.plan, self.pool, self.pool_s, w1, w1_scale, w2, w2_scale, epoch,
                               self.ws, self.y_pool, self.dtype, self.cfg, s)
            moe_combine(self.y_pool, topk_weights, self.plan, self.out, s)
            return self.out
        compute, comm = streams
        cur = torch.cuda.current_stream()
        comm.wait_stream(cur)
        moe_plan(topk_idx, self.plan, self.ws, comm)
        planned = torch.cuda.Event()
        planned.record(comm)
        moe_dispatch(x, self.plan, self.pool, self.pool_s, epoch, self.ws, self.dtype, comm)
        compute.wait_event(planned)
        ccfg = self._concurrent_cfg()
        if self.combine_on_completion:
            compute.wait_stream(cur)       # topk_weights and out belong to the caller's stream
            moe_expert_ffn_combine(self.plan, self.pool, self.pool_s, w1, w1_scale, w2, w2_scale, epoch,
                                   self.ws, self.y_pool, topk_weights, self.out, self.dtype, ccfg, compute)
            cur.wait_stream(compute)
            cur.wait_stream(comm)
            return self.out
        if self.train:
            moe_expert_ffn_train(self.plan, self.pool, w1, w2, epoch, self.ws, self.y_pool, self.g_pool,
                                 ccfg, compute)
        else:
            moe_expert_ffn(self.plan, self.pool, self.pool_s, w1, w1_scale, w2, w2_scale, epoch,
                           self.ws, self.y_pool, self.dtype, ccfg, compute)
        done = torch.cuda.Event()
        done.record(compute)
        comm.wait_event(done)
        moe_combine(self.y_pool, topk_weights, self.plan, self.out, comm)
        cur.wait_stream(comm)
        return self.out

    __call__ = forward


_LAYERS = {}


def stream_moe(x, topk_idx, topk_weights, w1_local, w2_local, *, expert_begin=0, tile=128,
               w1_scale=None, w2_scale=None, streams=None) -> torch.Tensor:
    """Functional form: shapes come from the tensors (w1_local [E_local, 2I, H]; uint8
    w1_local [E_local, 2I, H/2] means MXFP4). Returns a fresh output tensor; buffers are
    cached per shape and device."""
    T, H = x.shape
    K = topk_idx.shape[1]
    E, twoI, _ = w1_local.shape
    dtype = ("fp8" if w1_local.dtype == torch.float8_e4m3fn
             else "mxfp4" if w1_local.dtype == torch.uint8 else "bf16")
    key = (T, H, twoI // 2, K, E, expert_begin, tile, dtype, x.device)
    layer = _LAYERS.get(key)
    if layer is None:
        layer = StreamMoE(T, H, twoI // 2, K, E, expert_begin=expert_begin, tile=tile,
                          dtype=dtype, device=x.device)
        _LAYERS[key] = layer
    wkey = tuple((t.data_ptr(), t._version) if t is not None else None
                 for t in (w1_local, w2_local, w1_scale, w2_scale))
    if getattr(layer, "_wkey", None) != wkey:
        layer._wkey = wkey
        layer._w = layer.prepare_weights(w1_local, w2_local, w1_scale, w2_scale)
    w1p, w2p, s1p, s2p = layer._w
    out = layer.forward(x, topk_idx, topk_weights, w1p, w2p, s1p, s2p, streams)
    return out.clone()
