"""fp64 CPU reference of the multi-layer Performer language model on a whole
sequence (page "Sub-Linear Memory: How to Make Performers SLiM", Subsection 2.2:
the Transformer of eq. (5)-(9) with linear self-attention, and the next-token
loss (10)).  Its gradients are what the page's Algorithm 1 must reproduce.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use anything under oracle/.  This file shares no code with
the HIP path or its Python package: the architecture is written out here again,
plainly, and the attention runs in the fp64 C oracle (its masked quadratic form,
eq. (2)); the rest is ordinary PyTorch arithmetic on the CPU in float64, with
PyTorch's autograd as the chain rule.

Reading of the lost display equations (the same one the GPU path takes):
  X0_l = E[p_l] + pos(l), pos = sinusoids, positions l = 1..L;
  each layer: Xb = LN1(X); per head j the d columns j*d..(j+1)*d-1 of Xb W_Q,
  Xb W_K, Xb W_V are Q_j, K_j, V_j; X += concat_j Att^lin(Q_j, K_j, V_j);
  X += GeLU(LN2(X) W1 + b1) W2 + b2 (exact erf GeLU);
  logits = X W_out + b_out; loss = sum over l < L of cross entropy against p_{l+1}.
Parameters come in as the float32 arrays of synth.performer_params and are
widened exactly to float64.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import attn_bwd, attn_fwd


class _OracleAttention(torch.autograd.Function):
    """Att^lin (FAVOR+) by the oracle's quadratic form, q, k, v [B, H, L, d] float64;
    the gradient of the projection W too when it requires one."""

    @staticmethod
    def forward(ctx, q, k, v, W):
        ctx.save_for_backward(q, k, v, W)
        Y = attn_fwd(q.detach().numpy(), k.detach().numpy(), v.detach().numpy(), W.detach().numpy(), "favor",
                     form="quadratic")[0]
        return torch.from_numpy(Y)

    @staticmethod
    def backward(ctx, dY):
        q, k, v, W = ctx.saved_tensors
        want_dw = ctx.needs_input_grad[3]
        g = attn_bwd(q.detach().numpy(), k.detach().numpy(), v.detach().numpy(), W.detach().numpy(),
                     dY.detach().contiguous().numpy(), "favor", form="quadratic", want_dw=want_dw)
        dW = torch.from_numpy(g[5]) if want_dw else None
        return torch.from_numpy(g[0]), torch.from_numpy(g[1]), torch.from_numpy(g[2]), dW


def _positions(L: int, D: int) -> torch.Tensor:
    pe = torch.zeros((L, D), dtype=torch.float64)
    for l in range(1, L + 1):
        for i in range(0, D, 2):
            a = l / (10000.0 ** (i / D))
            pe[l - 1, i] = math.sin(a)
            pe[l - 1, i + 1] = math.cos(a)
    return pe


def _layer_norm(x, g, b, eps=1e-5):
    mu = x.mean(dim=-1, keepdim=True)
    var = ((x - mu) ** 2).mean(dim=-1, keepdim=True)
    return (x - mu) / torch.sqrt(var + eps) * g + b


def _gelu(x):
    return 0.5 * x * (1.0 + torch.erf(x / math.sqrt(2.0)))


def loss_and_grads(params: dict, tokens: np.ndarray, heads: int, layers: int, train_features: bool = False):
    """Loss (float) and {name: float64 gradient array} of every trainable
    parameter: all but the feature projections wf.r, which are fixed random
    draws unless train_features."""
    P = {n: torch.from_numpy(np.asarray(a, dtype=np.float64)).requires_grad_(train_features or
                                                                             not n.startswith("wf."))
         for n, a in params.items()}
    tok = torch.from_numpy(np.asarray(tokens, dtype=np.int64))
    B, L = tok.shape
    D = P["emb"].shape[1]
    d = D // heads
    X = P["emb"][tok] + _positions(L, D)[None]
    for r in range(layers):
        Xb = _layer_norm(X, P[f"ln1_g.{r}"], P[f"ln1_b.{r}"])

        def split(t):
            return t.reshape(B, L, heads, d).permute(0, 2, 1, 3).contiguous()
        Y = _OracleAttention.apply(split(Xb @ P[f"wq.{r}"]), split(Xb @ P[f"wk.{r}"]), split(Xb @ P[f"wv.{r}"]),
                                   P[f"wf.{r}"])
        X = X + Y.permute(0, 2, 1, 3).reshape(B, L, D)
        h = _layer_norm(X, P[f"ln2_g.{r}"], P[f"ln2_b.{r}"])
        X = X + _gelu(h @ P[f"w1.{r}"] + P[f"b1.{r}"]) @ P[f"w2.{r}"] + P[f"b2.{r}"]
    logits = X[:, :L - 1] @ P["wout"] + P["bout"]
    logp = logits - torch.logsumexp(logits, dim=-1, keepdim=True)
    loss = -logp.gather(-1, tok[:, 1:, None]).sum()
    loss.backward()
    return float(loss.detach()), {n: t.grad.numpy().copy() for n, t in P.items() if t.requires_grad}
