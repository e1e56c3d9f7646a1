"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module draws random numbers and nothing else: it holds none of the
attention arithmetic.  Both the HIP path and the CPU oracle receive exactly
the arrays produced here (after the same cast to the I/O dtype), so the two
sides can never disagree about an input.

Every per-head block of a [B, H, L, d] tensor comes from its own stream,
``PCG64(SeedSequence([seed, tensor_id, b, h]))``, so any single head can be
regenerated without drawing the rest (needed for the 1M-token workload).

For inputs too large to draw on the host in reasonable time (the 1M-token
workload), ``device_normal`` draws a whole [B, H, rows, cols] tensor from torch's
seeded device generator; the tests then copy the sampled heads of that very
tensor back for the oracle.

The FAVOR+ projection W ([M, d], one row per random feature) is also drawn
here: the feature map consumes it as an input.  Two draws are offered:
  * "gaussian":   iid N(0, 1) entries;
  * "orthogonal": ceil(M/d) independent d x d blocks, each the Q factor of a
    Gaussian QR with the sign of diag(R) folded in (a Haar-random orthogonal
    matrix); every row is then rescaled by the norm of an independent
    N(0, I_d) vector so that each row keeps the N(0, I_d) marginal.  The first
    M rows are kept.
"""
from __future__ import annotations

import numpy as np

# tensor ids of the per-head streams
TID_W, TID_Q, TID_K, TID_V, TID_DY, TID_R0, TID_S0, TID_DR, TID_DS = range(9)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, key)])))


def head_normal(seed: int, tid: int, b: int, h: int, rows: int, cols: int, scale: float) -> np.ndarray:
    """N(0, scale^2) float32 block [rows, cols] for head (b, h) of tensor `tid`."""
    x = _rng(seed, tid, b, h).standard_normal((rows, cols), dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def normal(seed: int, tid: int, B: int, H: int, rows: int, cols: int, scale: float) -> np.ndarray:
    """[B, H, rows, cols] float32, each head from its own stream."""
    out = np.empty((B, H, rows, cols), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            out[b, h] = head_normal(seed, tid, b, h, rows, cols, scale)
    return out


def device_normal(seed: int, tid: int, shape, scale: float, device="cuda"):
    """N(0, scale^2) float32 torch tensor of `shape` on `device`, from torch's
    generator seeded with (seed, tid)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + int(tid))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x


def positive(seed: int, tid: int, B: int, H: int, rows: int, cols: int, scale: float) -> np.ndarray:
    """[B, H, rows, cols] float32 drawn as scale * |N(0,1)| (for state tensors that
    must stay positive, e.g. a sum of positive features)."""
    return np.abs(normal(seed, tid, B, H, rows, cols, scale))


def projection(seed: int, M: int, d: int, kind: str = "gaussian") -> np.ndarray:
    """FAVOR+ projection W [M, d] float32 (see module docstring)."""
    g = _rng(seed, TID_W)
    if kind == "gaussian":
        return g.standard_normal((M, d)).astype(np.float32)
    if kind != "orthogonal":
        raise ValueError(kind)
    blocks = []
    for _ in range((M + d - 1) // d):
        A = g.standard_normal((d, d))
        q, r = np.linalg.qr(A)
        q = q * np.sign(np.diag(r))[None, :]
        blocks.append(q.T)  # rows orthonormal
    Wo = np.concatenate(blocks, axis=0)[:M]
    norms = np.linalg.norm(g.standard_normal((M, d)), axis=1)
    return np.ascontiguousarray((Wo * norms[:, None]).astype(np.float32))


# ---------------------------------------------------------------- model stack ---
# Randomly initialised parameters and random token strings for the multi-layer
# Performer stack (the page's experiments feed random strings to randomly
# initialised models).  Drawn here, in float32, so that the GPU path and the
# fp64 CPU reference receive the very same values.

TID_MODEL = 100


def performer_params(seed: int, vocab: int, d_model: int, heads: int, layers: int, M: int, d_ff: int) -> dict:
    """Parameters {name: float32 array} of an s-layer stack; layer r's names carry
    the suffix `.r`.  Matrices ~ N(0, 1/fan_in) (the query and key projections
    additionally times d^-1/4 with d = d_model / heads, which keeps g's arguments
    of order one), biases 0, layer-norm gains 1; `wf.r` [M, d] is layer r's fixed
    FAVOR+ projection, N(0, 1)."""
    d = d_model // heads
    g = _rng(seed, TID_MODEL)

    def mat(rows, cols, scale=1.0):
        return (g.standard_normal((rows, cols)) * (scale / np.sqrt(rows))).astype(np.float32)

    p = {"emb": (g.standard_normal((vocab, d_model)) * 0.5).astype(np.float32)}
    for r in range(layers):
        p[f"ln1_g.{r}"] = np.ones(d_model, np.float32)
        p[f"ln1_b.{r}"] = np.zeros(d_model, np.float32)
        p[f"wq.{r}"] = mat(d_model, d_model, d ** -0.25)
        p[f"wk.{r}"] = mat(d_model, d_model, d ** -0.25)
        p[f"wv.{r}"] = mat(d_model, d_model)
        p[f"ln2_g.{r}"] = np.ones(d_model, np.float32)
        p[f"ln2_b.{r}"] = np.zeros(d_model, np.float32)
        p[f"w1.{r}"] = mat(d_model, d_ff)
        p[f"b1.{r}"] = np.zeros(d_ff, np.float32)
        p[f"w2.{r}"] = mat(d_ff, d_model)
        p[f"b2.{r}"] = np.zeros(d_model, np.float32)
        p[f"wf.{r}"] = g.standard_normal((M, d)).astype(np.float32)
    p["wout"] = mat(d_model, vocab)
    p["bout"] = np.zeros(vocab, np.float32)
    return p


def random_tokens(seed: int, B: int, L: int, vocab: int) -> np.ndarray:
    """[B, L] int64 tokens drawn uniformly from the alphabet."""
    return _rng(seed, TID_MODEL + 1).integers(0, vocab, size=(B, L), dtype=np.int64)
