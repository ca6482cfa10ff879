"""CPU oracle of the MoE layer's backward pass -- test infrastructure only.

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
module. The GPU library never calls it and shares no code with it.

What it follows (StreamEP README, section "How it works"): the layer trains, and
besides the forward grouped GEMMs A and Y there are the backward grouped GEMMs A
and Y; the backward pass mirrors the forward's dispatch and combine. The page
gives no formulas, so the backward is the exact gradient of the forward the
oracle's moe_layer computes (bf16 mode, float64, no intermediate rounding):

  forward, per local pair q = (t, k) of expert e:
    G_q = x_t W1[e]^T,  g = G_q[:I], u = G_q[I:],  h_q = silu(g) * u,
    y_q = h_q W2[e]^T,  out_t = sum_k w[t,k] y_q
  backward, given dout [T, H]:
    dw[t,k]  = <dout_t, y_q>                   (0 for a non-local pair)
    dy_q     = w[t,k] dout_t                   (the combine's mirror: a scatter)
    dh_q     = dy_q W2[e]                      (backward GEMM Y, data gradient)
    dW2[e]   = sum_q dy_q^T h_q                (backward GEMM Y, weight gradient)
    dg       = dh * u * silu'(g),  du = dh * silu(g),
    silu'(z) = s(z) (1 + z (1 - s(z))),  s(z) = 1 / (1 + e^-z)
    dG_q     = [dg | du]
    dX_q     = dG_q W1[e]                      (backward GEMM A, data gradient)
    dW1[e]   = sum_q dG_q^T x_t                (backward GEMM A, weight gradient)
    dx_t     = sum_k dX_q                      (the dispatch's mirror: a gather-sum)

Readings where the page is silent: the gradient of topk_weights is returned (the
router trains through it); experts with no pair get zero weight gradients; the
pass is defined for the bf16 workloads (fp8 and MXFP4 are inference formats here).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .moe_oracle import _np, bf16_to_f64, expert_weights_f64, silu


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz [z * s(z)] = s(z) (1 + z (1 - s(z)))."""
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def expert_forward(X: np.ndarray, W1: np.ndarray, W2: np.ndarray):
    """(G, h, y) of one expert's rows, float64."""
    I = W1.shape[0] // 2
    G = X @ W1.T
    h = silu(G[:, :I]) * G[:, I:]
    return G, h, h @ W2.T


def expert_backward(X: np.ndarray, G: np.ndarray, h: np.ndarray, dy: np.ndarray, W1: np.ndarray,
                    W2: np.ndarray):
    """One expert's backward GEMMs Y and A: returns (dX [n, H], dW1 [2I, H], dW2 [H, I], dG [n, 2I])."""
    I = W1.shape[0] // 2
    g, u = G[:, :I], G[:, I:]
    dh = dy @ W2                       # backward Y, data
    dW2 = dy.T @ h                     # backward Y, weights
    dG = np.concatenate([dh * u * silu_grad(g), dh * silu(g)], axis=1)
    dX = dG @ W1                       # backward A, data
    dW1 = dG.T @ X                     # backward A, weights
    return dX, dW1, dW2, dG


@dataclass
class OracleGrads:
    dx: np.ndarray          # float64 [T, H]
    dw: np.ndarray          # float64 [T, K] (gradient of topk_weights)
    dW1: np.ndarray         # float64 [E_local, 2I, H]
    dW2: np.ndarray         # float64 [E_local, H, I]


def moe_layer_backward(inp, dout, experts: Optional[np.ndarray] = None) -> OracleGrads:
    """Gradients of the bf16 layer for the output gradient dout (bf16 or float [T, H]).
    ``experts`` restricts the weight gradients to those local experts (the data
    gradients then cover only their pairs)."""
    cfg = inp.cfg
    if cfg.dtype != "bf16":
        raise ValueError("the backward pass is defined for the bf16 workloads")
    ids = _np(inp.topk_idx).astype(np.int64)
    T, K = ids.shape
    E, H, I = cfg.num_local_experts, cfg.H, cfg.I
    w = _np(inp.topk_weights).astype(np.float64)
    x = bf16_to_f64(inp.x)
    d = dout if isinstance(dout, np.ndarray) else (
        bf16_to_f64(dout) if str(dout.dtype) == "torch.bfloat16" else _np(dout).astype(np.float64))
    d = np.asarray(d, dtype=np.float64)
    dx = np.zeros((T, H))
    dw = np.zeros((T, K))
    dW1 = np.zeros((E, 2 * I, H))
    dW2 = np.zeros((E, H, I))
    local_e = ids - cfg.expert_begin
    for e in (range(E) if experts is None else experts):
        tt, kk = np.nonzero(local_e == e)
        if tt.size == 0:
            continue
        W1, W2 = expert_weights_f64(inp.w1[e], None, inp.w2[e], None)
        X = x[tt]
        G, h, y = expert_forward(X, W1, W2)
        dw[tt, kk] = np.einsum("nh,nh->n", d[tt], y)
        dy = w[tt, kk][:, None] * d[tt]
        dX, dW1[e], dW2[e], _ = expert_backward(X, G, h, dy, W1, W2)
        np.add.at(dx, tt, dX)
    return OracleGrads(dx, dw, dW1, dW2)
