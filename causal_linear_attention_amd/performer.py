"""The page's memory-efficient training algorithm around the attention operation:
a multi-layer Performer trained slice by slice (page "Sub-Linear Memory: How to
Make Performers SLiM", Section 3, Algorithm 1).

The model (Subsection 2.2; its display equations did not survive extraction,
so the plainest GPT-2-like reading of the listed parameters is taken):

    X^(0)_l = emb(p_l) + pos(l)                      (sinusoidal positions, l = 1..L)
    for r = 1..s:   Xb = LN1(X);  per head j: Q_j, K_j, V_j = Xb W_Q, Xb W_K, Xb W_V
                    X  = X + concat_j Att^lin(Q_j, K_j, V_j)       (no output projection
                                                                    is listed, none is used)
                    X  = X + GeLU(LN2(X) W1 + b1) W2 + b2
    X^(out) = X^(s) W_out + b_out;   loss = sum_{l < L} CE(X^(out)_l, p_{l+1})

Att^lin is this package's causal linear attention (FAVOR+, one random
projection per layer, fixed as on the page or, with train_features, trained
through the backward's dW) and runs in the HIP kernels; everything else is
plain PyTorch (these layers are not the subject here).

Algorithm 1 (Subsection 3.2-3.3): the sequence is cut into N slices of length
at most C; the forward pass walks the slices in order, layers inside, carrying
only the per-layer attention states B = (R, S) across slices; the backward pass
walks the slices in reverse, rebuilds each slice's entry states by subtracting
the slice's own contributions from the exit states (update (19)), recomputes the
slice with autograd and back-propagates Phi^(n) = slice loss + <G^(n), B^(n)>,
which yields the slice's parameter gradients (accumulated into .grad) and the
gradient G^(n-1) of the entry states (update (20)).  Memory does not grow with
L beyond the token string and O(C) activations.
"""
from __future__ import annotations

import math

import torch
import torch.nn.functional as F

from . import attention as A
from . import synth


class _StatefulAttention(torch.autograd.Function):
    """Att^lin of one slice from an entry state: (q, k, v, R_in, S_in) ->
    (Y, R_out, S_out), with the backward through all five inputs (slim_attn_bwd
    with the incoming state gradient) and through W when it requires one."""

    @staticmethod
    def forward(ctx, q, k, v, R_in, S_in, W, num_chunks, state_dtype):
        Y, R, S, rs = A.attn_fwd(q, k, v, W, "favor", num_chunks, R_in=R_in, S_in=S_in, state_dtype=state_dtype,
                                 want_row_stats=True)
        ctx.save_for_backward(q, k, v, W, R_in if R_in is not None else torch.empty(0),
                              S_in if S_in is not None else torch.empty(0), Y, rs)
        ctx.has_state = R_in is not None
        ctx.num_chunks, ctx.state_dtype = num_chunks, R.dtype
        return Y, R, S

    @staticmethod
    def backward(ctx, dY, dR, dS):
        q, k, v, W, R_in, S_in, Y, rs = ctx.saved_tensors
        if dY is None:
            dY = torch.zeros_like(q)
        sd = ctx.state_dtype
        if dR is None and dS is not None:
            dR = torch.zeros((q.shape[0], q.shape[1], q.shape[3], W.shape[0]), dtype=sd, device=q.device)
        if dS is None and dR is not None:
            dS = torch.zeros((q.shape[0], q.shape[1], W.shape[0]), dtype=sd, device=q.device)
        st = (R_in, S_in) if ctx.has_state else (None, None)
        want_dw = ctx.needs_input_grad[5]
        g = A.attn_bwd(q, k, v, W, dY.contiguous(), "favor", ctx.num_chunks, R_in=st[0], S_in=st[1], dR_out=dR,
                       dS_out=dS, want_state_grad=ctx.has_state, state_dtype=sd, want_dw=want_dw, Y=Y,
                       row_stats=rs)
        dW = g[5].to(W.dtype) if want_dw else None
        return g[0], g[1], g[2], g[3], g[4], dW, None, None


def sinusoid(positions: torch.Tensor, d_model: int) -> torch.Tensor:
    """Sinusoidal position embedding of the given 1-based positions [n] -> [n, d_model]."""
    i = torch.arange(0, d_model, 2, device=positions.device, dtype=torch.float32)
    ang = positions.to(torch.float32)[:, None] / torch.pow(10000.0, i / d_model)[None, :]
    pe = torch.empty((positions.shape[0], d_model), device=positions.device)
    pe[:, 0::2] = torch.sin(ang)
    pe[:, 1::2] = torch.cos(ang)
    return pe


class Performer:
    """A randomly initialised s-layer Performer (parameters from synth.performer_params)."""

    def __init__(self, vocab=64, d_model=64, heads=2, layers=2, M=64, d_ff=None, seed=0, device="cuda",
                 num_chunks=1, state_dtype=torch.float64, train_features=False):
        self.vocab, self.d_model, self.heads, self.layers, self.M = vocab, d_model, heads, layers, M
        self.d = d_model // heads
        self.d_ff = d_ff or 4 * d_model
        self.num_chunks = num_chunks  # slices of the attention op inside one call
        # type of the attention states carried between slices: fp64 (the op's internal
        # carry precision) by default, so that the slice boundaries add no rounding
        self.state_dtype = state_dtype
        raw = synth.performer_params(seed, vocab, d_model, heads, layers, M, self.d_ff)
        self.p = {}
        for n, a in raw.items():
            t = torch.from_numpy(a).to(device)
            if train_features or not n.startswith("wf."):  # wf.r: the layers' feature projections
                t.requires_grad_(True)
            self.p[n] = t

    def parameters(self):
        return {n: t for n, t in self.p.items() if t.requires_grad}

    def zero_grad(self):
        for t in self.parameters().values():
            t.grad = None

    # -- the rowwise parts (F and G of the page's compact form) --
    def embed(self, tokens, start):
        pos = torch.arange(start + 1, start + 1 + tokens.shape[1], device=tokens.device)
        return self.p["emb"][tokens] + sinusoid(pos, self.d_model)[None]

    def qkv(self, r, X):
        p, B, L = self.p, X.shape[0], X.shape[1]
        Xb = F.layer_norm(X, (self.d_model,), p[f"ln1_g.{r}"], p[f"ln1_b.{r}"])

        def heads(t):
            return t.view(B, L, self.heads, self.d).transpose(1, 2).contiguous()
        return heads(Xb @ p[f"wq.{r}"]), heads(Xb @ p[f"wk.{r}"]), heads(Xb @ p[f"wv.{r}"])

    def finish(self, r, X, Y):
        p, B, L = self.p, X.shape[0], X.shape[1]
        X = X + Y.transpose(1, 2).reshape(B, L, self.d_model)
        h = F.layer_norm(X, (self.d_model,), p[f"ln2_g.{r}"], p[f"ln2_b.{r}"])
        return X + F.gelu(h @ p[f"w1.{r}"] + p[f"b1.{r}"]) @ p[f"w2.{r}"] + p[f"b2.{r}"]

    def layer(self, r, X, R_in=None, S_in=None):
        q, k, v = self.qkv(r, X)
        Y, R, S = _StatefulAttention.apply(q, k, v, R_in, S_in, self.p[f"wf.{r}"], self.num_chunks,
                                           self.state_dtype)
        return self.finish(r, X, Y), R, S

    def slice_loss(self, X, tokens, a, b):
        """Summed next-token cross entropy of positions a..b-1 (the last position of
        the sequence has no target)."""
        L = tokens.shape[1]
        n = min(b, L - 1) - a
        if n <= 0:
            return X.sum() * 0.0
        logits = X[:, :n] @ self.p["wout"] + self.p["bout"]
        return F.cross_entropy(logits.reshape(-1, self.vocab), tokens[:, a + 1:a + 1 + n].reshape(-1),
                               reduction="sum")

    # -- evaluation strategies --
    def loss_full(self, tokens):
        """The whole sequence in one pass (C = L); differentiable by autograd."""
        X = self.embed(tokens, 0)
        for r in range(self.layers):
            X, _, _ = self.layer(r, X)
        return self.slice_loss(X, tokens, 0, tokens.shape[1])

    def algorithm1(self, tokens, C):
        """Loss and parameter gradients (accumulated into .grad) by the page's
        Algorithm 1 with slices of length at most C.  Returns the loss."""
        L = tokens.shape[1]
        N = math.ceil(L / C)
        bounds = [(n * C, min(L, (n + 1) * C)) for n in range(N)]
        # forward: slices outer, layers inner; only the states B cross slices
        states = [(None, None)] * self.layers
        loss = 0.0
        with torch.no_grad():
            for a, b in bounds:
                X = self.embed(tokens[:, a:b], a)
                for r in range(self.layers):
                    X, R, S = self.layer(r, X, *states[r])
                    states[r] = (R, S)
                loss += float(self.slice_loss(X, tokens, a, b))
        # backward: slices in reverse; B^(n) known, G^(N) = 0
        Bn = [(R.double(), S.double()) for R, S in states]
        G = [(torch.zeros_like(R), torch.zeros_like(S)) for R, S in states]
        for a, b in reversed(bounds):
            X = self.embed(tokens[:, a:b], a)
            entry, exits = [], []
            for r in range(self.layers):
                q, k, v = self.qkv(r, X)
                with torch.no_grad():  # this slice's own contribution to layer r's state
                    _, dR, dS = A.attn_fwd(q.detach(), k.detach(), v.detach(), self.p[f"wf.{r}"], "favor",
                                           self.num_chunks, state_dtype=self.state_dtype)
                # update (19): entry state = exit state minus the slice's contribution
                R_in = (Bn[r][0] - dR.double()).to(dR.dtype).requires_grad_(True)
                S_in = (Bn[r][1] - dS.double()).to(dS.dtype).requires_grad_(True)
                Y, R, S = _StatefulAttention.apply(q, k, v, R_in, S_in, self.p[f"wf.{r}"], self.num_chunks,
                                                   self.state_dtype)
                X = self.finish(r, X, Y)
                entry.append((R_in, S_in))
                exits.append((R, S))
            phi = self.slice_loss(X, tokens, a, b)
            for (R, S), (gR, gS) in zip(exits, G):
                phi = phi + (R * gR).sum() + (S * gS).sum()
            phi.backward()
            # update (20): the entry states' gradient is the next (earlier) slice's G
            G = [(R_in.grad.detach(), S_in.grad.detach()) for R_in, S_in in entry]
            Bn = [(R_in.detach().double(), S_in.detach().double()) for R_in, S_in in entry]
        return loss
