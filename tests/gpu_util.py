"""Shared helpers of the GPU parity tests: seeded inputs (from the shared
generator), the oracle's answer on exactly the values the GPU received, and
the normwise error metric."""
from __future__ import annotations

import numpy as np
import torch

from causal_linear_attention_amd import synth

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_dev(x: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def host64(t: torch.Tensor) -> np.ndarray:
    # widened on the host: an fp64 tensor keeps every bit
    return t.detach().cpu().double().numpy()


def inputs(B, H, L, d, M, dtype, feat="favor", seed=0, scale=None, w_kind="gaussian", dy=True):
    """Device tensors (io dtype) for Q, K, V, W, dY drawn by the shared generator."""
    scale = d ** -0.25 if scale is None else scale
    t = dict(
        q=to_dev(synth.normal(seed, synth.TID_Q, B, H, L, d, scale), dtype),
        k=to_dev(synth.normal(seed, synth.TID_K, B, H, L, d, scale), dtype),
        v=to_dev(synth.normal(seed, synth.TID_V, B, H, L, d, 1.0), dtype),
        W=to_dev(synth.projection(seed, M, d, w_kind), dtype) if feat == "favor" else None,
    )
    if dy:
        t["dy"] = to_dev(synth.normal(seed, synth.TID_DY, B, H, L, d, 1.0), dtype)
    return t


def relerr_heads(got, ref) -> float:
    """max over (b, h) of ||got - ref||_2 / ||ref||_2 (normwise, per head)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    g = g.reshape(g.shape[0] * g.shape[1], -1)
    r = r.reshape(r.shape[0] * r.shape[1], -1)
    num = np.linalg.norm(g - r, axis=1)
    den = np.maximum(np.linalg.norm(r, axis=1), 1e-300)
    return float(np.max(num / den))


def relerr(got, ref) -> float:
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
