"""Shared helpers of the GPU parity tests: seeded inputs (from the shared
generator), the oracle's answer on exactly the values the GPU received, and
the error metrics.

Metrics (per (batch, head), maximum over heads), each with its own bound:
  * normwise relative error ||x - x_ref|| / ||x_ref|| (the page's gradient
    discrepancy metric, experiments section): below tol (1e-4 fp32, 2e-2 bf16);
  * max-abs / max-ref, max |x - x_ref| / max |x_ref| over the head: below
    MAXABS_FACTOR * tol;
  * worst row: max over rows l of ||x_l - x_ref,l|| / max(||x_ref,l||, rms),
    rms = the head's root-mean-square row norm (a row above that size against
    its own norm, a smaller one against it): below ROW_FACTOR * tol.  A wrong
    row of typical size gives about 1 here while adding only 1/sqrt(rows) to
    the normwise error;
  * positional classes (when the slice length c and tile rows TT are given):
    for each class of rows that one kind of boundary bug would hit together --
    the rows at each position 0..TT-1 of their tile, the first and the last row
    of every slice, the rows of each slice's partial last tile, the rows of a
    shorter last slice -- the error ||x_c - x_ref,c|| / max(||x_ref,c||,
    rms sqrt(n_c)) over its n_c rows, below tol * max(CLASS_FACTOR,
    ROW_FACTOR / sqrt(n_c)) (a class may hold one row of the worst-row bound; a
    large class must average out like a head).  A systematic slice-boundary or
    ragged-tile error of typical size gives about 1 for its class, far above
    that bound for any n_c.
Why these bounds.  The bf16 operands of the products carry a relative rounding
of up to 2^-9 each.  Averaged over a head this gives the normwise 3e-3..8e-3
measured; the worst element and the worst row are the tail of that
distribution.  Y, dV, the states and dW keep it short (worst rows within 2e-2
of their size).  dQ and dK, the outputs of the FAVOR+ chain rule, have a long
tail: a dQ row is a difference of terms that cancel (sum over s of
A[t][s] P[t][s] is exactly 0), and a dK row is a sum over all later queries of
terms of both signs that can be small by chance; either way a row can be much
smaller than the terms that make it and still carry their rounding.  Emulating
the kernels' bf16 roundings in fp64 on the CPU reproduces it: the worst dQ row
at 0.04 to 0.07 of a typical row at 4096 rows, with no single dominant source
(dNum, dden, Y, the state copy and g(K) contribute alike), the worst dK row
driven by the rounding of dNum.  The tail grows with the number of rows looked
at: on the GPU the worst of 2^20 rows (the 1M-token workload) reaches 0.39 of
the RMS row norm (dK) and 0.27 (dQ).  Hence 25 x tol per row.  The worst
element of a head stays below 2 x tol, and so does every positional class (a
class of a few hundred rows averages the tail out like a head does).  fp32
results sit at 1e-6..1e-5 of the oracle, so the same factors hold there with
room to spare.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

from causal_linear_attention_amd import synth

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DT = {"f32": torch.float32, "bf16": torch.bfloat16}
ROW_FACTOR = 25.0
MAXABS_FACTOR = 2.0
CLASS_FACTOR = 2.0
KOFF_MARGIN = 60.0  # the key-side offset's margin (include/slim.h)


def koff_of(W) -> float:
    """The key-side offset of W by its definition, max(0, max_m |w_m|^2/2 - 60), in fp64."""
    if W is None:
        return 0.0
    w = W.detach().cpu().double().numpy() if hasattr(W, "detach") else np.asarray(W, dtype=np.float64)
    return max(0.0, float(np.max(np.sum(w * w, axis=1))) / 2.0 - KOFF_MARGIN)


def position_classes(L: int, c: int, tt: int) -> dict:
    """{name: row indices} of the rows a boundary bug would hit together (see the
    module docstring), for a sequence of L rows cut into slices of c rows walked in
    tiles of tt rows."""
    rows = np.arange(L)
    ins = rows % c
    cls = {f"tile row {j}": rows[ins % tt == j] for j in range(tt)}
    cls["slice first"] = rows[ins == 0]
    cls["slice last"] = rows[(ins == c - 1) | (rows == L - 1)]
    if c % tt:
        cls["partial tile"] = rows[ins >= (c // tt) * tt]
    last = (L - 1) // c * c
    if L - last < c:
        cls["short last slice"] = rows[last:]
        if (L - last) % tt:
            cls["partial tile of the last slice"] = rows[last + (L - last) // tt * tt:]
    return {k: v for k, v in cls.items() if v.size}


def metrics(got, ref, rows_axis=True, positions=None) -> dict:
    """{"norm", "maxabs", "row"[, "class", "worst class"]} of got against ref, each the
    maximum over the leading (batch, head) pairs; rows are the second-to-last axis
    (rows_axis=False: the whole head is one row).  positions = (c, tt): also the
    normwise error of each positional class of rows."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.ndim >= 3:  # [B, H, ...]: one head per (b, h)
        nh = g.shape[0] * g.shape[1]
        cols = g.shape[-1] if rows_axis else int(np.prod(g.shape[2:]))
    else:  # one matrix (or vector): a single "head"
        nh = 1
        cols = g.shape[-1] if (rows_axis and g.ndim == 2) else g.size
    g = g.reshape(nh, -1, cols)
    r = r.reshape(g.shape)
    e = g - r
    norm = np.linalg.norm(e.reshape(nh, -1), axis=1) / np.maximum(np.linalg.norm(r.reshape(nh, -1), axis=1), 1e-300)
    maxabs = np.abs(e).reshape(nh, -1).max(axis=1) / np.maximum(np.abs(r).reshape(nh, -1).max(axis=1), 1e-300)
    rn = np.linalg.norm(r, axis=2)
    rms = np.sqrt(np.mean(rn * rn, axis=1, keepdims=True))
    row = (np.linalg.norm(e, axis=2) / np.maximum(np.maximum(rn, rms), 1e-300)).max(axis=1)
    out = {"norm": float(norm.max()), "maxabs": float(maxabs.max()), "row": float(row.max())}
    if positions is not None:
        c, tt = positions
        worst, name = 0.0, None
        for k, idx in position_classes(g.shape[1], c, tt).items():
            n = idx.size
            ec = np.linalg.norm(e[:, idx].reshape(nh, -1), axis=1)
            rc = np.maximum(np.linalg.norm(r[:, idx].reshape(nh, -1), axis=1), rms[:, 0] * np.sqrt(n))
            # the class error in units of tol's share: below tol when within its bound
            v = float((ec / np.maximum(rc, 1e-300)).max()) / max(CLASS_FACTOR, ROW_FACTOR / np.sqrt(n))
            if v > worst:
                worst, name = v, k
        out["class"], out["worst class"] = worst, name
    return out


def check(what, got, ref, tol, rows_axis=True, positions=None) -> dict:
    """Assert every metric against its bound (see the module docstring).  positions =
    (slice length, tile rows) of the run adds the positional classes.  With
    SLIM_PARITY_LOG set, each check is appended to that file as a JSON line."""
    m = metrics(got, ref, rows_axis, positions)
    path = os.environ.get("SLIM_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"what": str(what), "tol": tol, **m}) + "\n")
    assert m["norm"] < tol, (what, "normwise", m)
    assert m["maxabs"] < MAXABS_FACTOR * tol, (what, "max-abs/max-ref", m)
    assert m["row"] < ROW_FACTOR * tol, (what, "worst row", m)
    if positions is not None:
        assert m["class"] < tol, (what, "positional class", m)
    return m


def tile_rows(q, M, feat, C) -> int:
    """Rows per tile of the chunk kernels for this call's shape (slim_tile_rows)."""
    import ctypes

    from causal_linear_attention_amd import _lib
    from causal_linear_attention_amd import attention as A
    return int(_lib.lib().slim_tile_rows(ctypes.byref(A.make_desc(q, M, feat, C))))


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


def gpu_koff(W) -> float:
    """The key-side offset the library computes for W (one tiny forward); 0 without W."""
    if W is None:
        return 0.0
    from causal_linear_attention_amd import attention as A
    M, d = W.shape
    x = torch.zeros((1, 1, 1, d), dtype=W.dtype, device=W.device)
    ko = torch.full((1,), -1.0, device=W.device)
    A.attn_fwd(x, x, x, W, "favor", 1, koff_out=ko)
    k = float(ko)
    assert abs(k - koff_of(W)) <= 1e-5 * max(1.0, k), (k, koff_of(W))
    return k
