"""Pins of the oracle's backward pass (no GPU).

* every gradient (dx, topk_weights, dW1, dW2) equals torch.autograd's on the same
  float64 forward built from torch.nn.functional (a library differentiation,
  independent of the oracle's hand-derived formulas), including non-local ids and
  an expert with no pair;
* silu' equals a central finite difference;
* with one expert, K = 1 and weight 1, dW1 / dW2 equal the textbook dense-MLP
  gradients (a plain formula on the whole batch).
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
from synth import MoEConfig, make_dout, make_inputs


def _autograd(inp, dout):
    cfg = inp.cfg
    x = torch.from_numpy(oracle.bf16_to_f64(inp.x))
    w = inp.topk_weights.double().clone().requires_grad_(True)
    W1 = torch.from_numpy(np.stack([oracle.bf16_to_f64(inp.w1[e]) for e in range(cfg.num_local_experts)]))
    W2 = torch.from_numpy(np.stack([oracle.bf16_to_f64(inp.w2[e]) for e in range(cfg.num_local_experts)]))
    W1.requires_grad_(True)
    W2.requires_grad_(True)
    x.requires_grad_(True)
    idx = inp.topk_idx.long() - cfg.expert_begin
    out = torch.zeros(cfg.T, cfg.H, dtype=torch.float64)
    for k in range(cfg.K):
        for e in range(cfg.num_local_experts):
            m = idx[:, k] == e
            if not bool(m.any()):
                continue
            G = F.linear(x[m], W1[e])
            h = F.silu(G[:, :cfg.I]) * G[:, cfg.I:]
            y = F.linear(h, W2[e])
            out = out.index_add(0, m.nonzero().squeeze(1), w[m, k:k + 1] * y)
    out.backward(torch.from_numpy(oracle.bf16_to_f64(dout)))
    return x.grad.numpy(), w.grad.numpy(), W1.grad.numpy(), W2.grad.numpy()


def _close(a, b, tol=1e-11):
    scale = max(np.abs(b).max(), 1e-300)
    assert np.abs(a - b).max() <= tol * scale, (np.abs(a - b).max(), scale)


def test_backward_matches_autograd_with_nonlocal_and_empty_expert():
    cfg = MoEConfig("bwd_small", 24, 32, 16, 7, 2, 4, 3, 4)       # experts 2..5 local of 7
    inp = make_inputs(cfg, 11)
    idx = inp.topk_idx.clone()
    idx[idx == 4] = 6                                                # local expert 2 gets no pair
    inp = inp.__class__(**{**inp.__dict__, "topk_idx": idx})
    dout = make_dout(cfg, 11)
    g = oracle.moe_layer_backward(inp, dout)
    dx, dw, dW1, dW2 = _autograd(inp, dout)
    _close(g.dx, dx)
    _close(g.dw, dw)
    _close(g.dW1, dW1)
    _close(g.dW2, dW2)
    assert not g.dW1[2].any() and not g.dW2[2].any()
    nonlocal_pairs = (idx < 2) | (idx >= 6)
    assert (g.dw[nonlocal_pairs.numpy()] == 0).all()


def test_silu_grad_finite_difference():
    z = np.linspace(-12, 12, 97)
    eps = 1e-6
    fd = (oracle.silu(z + eps) - oracle.silu(z - eps)) / (2 * eps)
    assert np.abs(oracle.silu_grad(z) - fd).max() < 1e-8
    assert oracle.silu_grad(np.array([0.0]))[0] == 0.5


def test_dense_mlp_weight_gradients():
    cfg = MoEConfig("bwd_dense", 9, 16, 8, 1, 0, 1, 1, 1)
    inp = make_inputs(cfg, 3)
    inp = inp.__class__(**{**inp.__dict__, "topk_weights": torch.ones(9, 1)})
    dout = make_dout(cfg, 3)
    g = oracle.moe_layer_backward(inp, dout)
    X = oracle.bf16_to_f64(inp.x)
    W1 = oracle.bf16_to_f64(inp.w1[0])
    W2 = oracle.bf16_to_f64(inp.w2[0])
    D = oracle.bf16_to_f64(dout)
    A = X @ W1.T
    a, b = A[:, :8], A[:, 8:]
    sg = 1 / (1 + np.exp(-a))
    H_ = a * sg * b
    dH = D @ W2
    dA = np.concatenate([dH * b * (sg + a * sg * (1 - sg)), dH * a * sg], axis=1)
    _close(g.dW2[0], D.T @ H_)
    _close(g.dW1[0], dA.T @ X)
    _close(g.dx, dA @ W1)
