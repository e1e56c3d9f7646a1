"""GPU against the fp64 oracle at the full sizes of the five measured workloads,
in the launch configuration bench.py times (same slice counts, automatic
window), through the C ABI.  The oracle evaluates sampled heads completely
(its linear-time prefix form, itself pinned against the quadratic definition);
the 1M-token workload is checked on what the oracle can evaluate at that size:
  * causality: with dY = 0 past row L', rows < L' of Y, dQ, dK, dV equal the
    oracle on the first L' rows, and rows >= L' of dQ, dK, dV are exactly 0;
  * the final state R_out = sum_i V_i g(K_i)^T, S_out = sum_i g(K_i) over all
    1M rows equals the oracle's feature map summed with a matrix product.
Inputs come from the seeded device generator (synth.device_normal); the oracle
receives the sampled heads of those same device tensors.  Tolerance: normwise
relative error per head, 1e-4 for fp32, 2e-2 for bf16."""
import numpy as np
import pytest
import torch

import oracle
from causal_linear_attention_amd import attention as A
from causal_linear_attention_amd import synth
from causal_linear_attention_amd.workloads import WORKLOADS
from gpu_util import DT, TOL, host64, relerr

pytestmark = pytest.mark.gpu


def make(w, dy=True):
    dt = DT[w.dtype]
    shp = (w.B, w.H, w.L, w.d)
    x = {
        "q": synth.device_normal(w.seed, synth.TID_Q, shp, w.qkv_scale).to(dt),
        "k": synth.device_normal(w.seed, synth.TID_K, shp, w.qkv_scale).to(dt),
        "v": synth.device_normal(w.seed, synth.TID_V, shp, 1.0).to(dt),
        "W": None,
    }
    if w.feat == "favor":
        x["W"] = torch.from_numpy(synth.projection(w.seed, w.M, w.d, w.w_kind)).to(dt).cuda()
    if dy:
        x["dy"] = synth.device_normal(w.seed, synth.TID_DY, shp, 1.0).to(dt)
    return x


def heads(t, sel, rows=None):
    """fp64 host copy [1, len(sel), rows, ...] of the selected (b, h) heads."""
    out = [host64(t[b, h] if rows is None else t[b, h, :rows]) for b, h in sel]
    return np.stack(out)[None]


@pytest.mark.parametrize("name", ["favor_ortho_f32_L4096_d64_M128", "favor_bf16_L16384_d64_M256",
                                  "elu1_bf16_L8192_d128"])
def test_fullsize_fwd_bwd_sampled_heads(name):
    w = WORKLOADS[name]
    print("fullsize", name, flush=True)
    x = make(w)
    # as the bench step runs it: the forward keeps its row statistics for the backward
    Y, R, S, rs = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], w.feat, w.chunks, want_row_stats=True)
    dQ, dK, dV, _, _ = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], w.feat, w.chunks, Y=Y, row_stats=rs)
    # and the backward that recomputes them
    dQ0, dK0, dV0, _, _ = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], w.feat, w.chunks)
    torch.cuda.synchronize()
    sel = [(0, 0), (w.B - 1, w.H - 1)]
    Wh = None if x["W"] is None else host64(x["W"])
    q, k, v, dy = (heads(x[n], sel) for n in ("q", "k", "v", "dy"))
    Yo, _, Ro, So = oracle.attn_fwd(q, k, v, Wh, w.feat, form="prefix")
    gq, gk, gv, _, _ = oracle.attn_bwd(q, k, v, Wh, dy, w.feat, form="prefix")
    tol = TOL[DT[w.dtype]]
    for i, (b, h) in enumerate(sel):
        for nm, got, ref in (("Y", Y, Yo), ("R", R, Ro), ("S", S, So), ("dQ", dQ, gq), ("dK", dK, gk),
                             ("dV", dV, gv), ("dQ recomputed statistics", dQ0, gq),
                             ("dK recomputed statistics", dK0, gk), ("dV recomputed statistics", dV0, gv)):
            e = relerr(host64(got[b, h]), ref[0, i])
            assert e < tol, (name, (b, h), nm, e)
    for t in (Y, dQ, dK, dV):
        assert torch.isfinite(t).all()


def test_fullsize_long_context_causal_prefix_and_final_state():
    w = WORKLOADS["favor_bf16_L1048576_d64_M64"]
    Lp = 32768
    print("fullsize", w.name, "L'", Lp, flush=True)
    x = make(w)
    x["dy"][:, :, Lp:] = 0
    Y, R, S, rs = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], w.feat, w.chunks, want_row_stats=True)
    dQ, dK, dV, _, _ = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], w.feat, w.chunks, Y=Y, row_stats=rs)
    torch.cuda.synchronize()
    # rows past L' receive no gradient at all
    for nm, t in (("dQ", dQ), ("dK", dK), ("dV", dV)):
        assert int(torch.count_nonzero(t[:, :, Lp:])) == 0, nm
        assert torch.isfinite(t).all(), nm
    assert torch.isfinite(Y).all()
    sel = [(0, w.H - 1)]
    Wh = host64(x["W"])
    q, k, v, dy = (heads(x[n], sel, Lp) for n in ("q", "k", "v", "dy"))
    Yo, _, _, _ = oracle.attn_fwd(q, k, v, Wh, w.feat, form="prefix")
    gq, gk, gv, _, _ = oracle.attn_bwd(q, k, v, Wh, dy, w.feat, form="prefix")
    tol = TOL[DT[w.dtype]]
    b, h = sel[0]
    for nm, got, ref in (("Y", Y, Yo), ("dQ", dQ, gq), ("dK", dK, gk), ("dV", dV, gv)):
        e = relerr(host64(got[b, h, :Lp]), ref[0, 0])
        assert e < tol, (nm, e)
    # final state over all 1M rows: R[e][m] = sum_i V_i[e] g(K_i)[m], S = sum_i g(K_i)
    kf, vf = host64(x["k"][b, h]), host64(x["v"][b, h])
    phi = oracle.featmap(kf[None, None], Wh, w.feat)[0, 0]
    assert relerr(host64(R[b, h]), vf.T @ phi) < tol
    assert relerr(host64(S[b, h]), phi.sum(axis=0)) < tol


def test_fullsize_featmap_sampled_rows():
    # the standalone feature map on the headline workload's Q (1M rows, as bench.py
    # --featmap times it): sampled rows, including every workgroup boundary of the first
    # few and the last rows, against the oracle's features
    w = WORKLOADS["favor_bf16_L16384_d64_M256"]
    x = make(w, dy=False)
    phi, off = A.featmap(x["q"], x["W"], "favor", row_offset=True)
    torch.cuda.synchronize()
    rows = w.B * w.H * w.L
    sel = np.unique(np.concatenate([np.arange(0, 1024, 31), [255, 256, 257, rows - 257, rows - 256, rows - 1],
                                    np.random.default_rng(3).integers(0, rows, 500)]))
    qf = x["q"].reshape(rows, w.d)[torch.from_numpy(sel).cuda()]
    ref = oracle.featmap(host64(qf), host64(x["W"]), "favor")
    got = host64(phi.reshape(rows, w.M)[torch.from_numpy(sel).cuda()])
    o = host64(off.reshape(rows)[torch.from_numpy(sel).cuda()])
    assert relerr(got * np.exp(o)[:, None], ref) < 1e-5
    assert float(got.max()) <= 1.0 / np.sqrt(w.M) * (1 + 1e-5)  # the offset makes the largest feature 1/sqrt(M)
    assert torch.isfinite(phi).all()
