"""Groups of slices (slim_desc.group_slices): one workgroup walks G consecutive
slices, carrying the state from one to the next, as the page's slice loop carries
it (page "Sub-Linear Memory: How to Make Performers SLiM", Subsection 3.2); one state
per group is stored, scanned and (backward) read back.  The grouping changes only
the fp32 rounding order, so every grouping is held to the oracle at the usual bounds,
including the row statistics kernel, which splits a group into parts of 256 rows:
  * given groups (2, 3, 5 slices, the last group short or a single slice), with an
    initial state and incoming state gradients, the forward's row statistics and
    kept states, and dW;
  * several windows of groups (a window given in slices holds whole groups);
  * the automatic grouping where it walks four slices per workgroup, against one
    slice per workgroup and the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from causal_linear_attention_amd import _lib
from causal_linear_attention_amd import attention as A
from gpu_util import DT, TOL, check, gpu_koff, host64, inputs, tile_rows

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, L, d, M, slices, group, dtype, feat
    (1, 2, 1000, 64, 128, 8, 2, "f32", "favor"),   # slices of 125: groups of 250, last one short
    (1, 2, 2100, 64, 256, 7, 3, "bf16", "favor"),  # slices of 300: groups of 900 (four row-statistics parts)
    (2, 1, 700, 32, 32, 9, 5, "f32", "elu1"),      # slices of 78: 2 groups, the second of 4 slices
    (1, 2, 1536, 128, 128, 6, 2, "bf16", "elu1"),
    (2, 2, 1500, 64, 64, 7, 2, "bf16", "favor"),   # slices of 215: the shared-operand dK path
]


def _id(c):
    return "B%dH%dL%d_d%dM%d_C%d_G%d_%s_%s" % c


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_groups_against_the_oracle(case):
    B, H, L, d, M, C, G, dt, feat = case
    dtype = DT[dt]
    x = inputs(B, H, L, d, M, dtype, feat, seed=91)
    dsc = A.make_desc(x["q"], M, feat, C, group_slices=G)
    assert _lib.lib().slim_group_slices(ctypes.byref(dsc)) == G
    rng = np.random.default_rng(92)
    R0 = torch.from_numpy(rng.random((B, H, d, M)).astype(np.float32)).cuda()
    S0 = torch.from_numpy(rng.random((B, H, M)).astype(np.float32)).cuda()
    dR = torch.from_numpy(rng.standard_normal((B, H, d, M)).astype(np.float32)).cuda()
    dS = torch.from_numpy(rng.standard_normal((B, H, M)).astype(np.float32)).cuda()
    print("groups", _id(case), flush=True)
    q, k, v, W, dy = x["q"], x["k"], x["v"], x["W"], x["dy"]
    Y, R, S, rs, st = A.attn_fwd(q, k, v, W, feat, C, R_in=R0, S_in=S0, want_row_stats=True, want_states=True,
                                 group_slices=G)
    kw = dict(R_in=R0, S_in=S0, dR_out=dR, dS_out=dS, want_state_grad=True, want_dw=feat == "favor",
              group_slices=G)
    g = A.attn_bwd(q, k, v, W, dy, feat, C, Y=Y, row_stats=rs, states=st, **kw)
    g1 = A.attn_bwd(q, k, v, W, dy, feat, C, Y=Y, row_stats=rs, **kw)  # rebuilding the states
    g0 = A.attn_bwd(q, k, v, W, dy, feat, C, **kw)  # rebuilding states and statistics
    torch.cuda.synchronize()
    cs = -(-L // C)
    assert st is not None and st.shape[2] == -(-L // min(cs * G, L)) + 1
    for a, b in zip(g, g1):
        assert torch.equal(a, b)
    h = {n: host64(x[n]) for n in ("q", "k", "v", "dy")}
    Wh = host64(W) if feat == "favor" else None
    e = np.exp(gpu_koff(W)) if feat == "favor" else 1.0
    Yo, _, Ro, So = oracle.attn_fwd(h["q"], h["k"], h["v"], Wh, feat, R0=host64(R0) * e, S0=host64(S0) * e,
                                    form="prefix")
    o = oracle.attn_bwd(h["q"], h["k"], h["v"], Wh, h["dy"], feat, R0=host64(R0) * e, S0=host64(S0) * e,
                        dRout=host64(dR) / e, dSout=host64(dS) / e, form="prefix", want_dw=feat == "favor")
    tol = TOL[dtype]
    pos = (min(cs * G, L), tile_rows(q, M, feat, C))
    check(("groups Y", _id(case)), host64(Y), Yo, tol, positions=pos)
    check(("groups R", _id(case)), host64(R) * e, Ro, tol)
    check(("groups S", _id(case)), host64(S) * e, So, tol)
    for name, a, a0, ref in zip(("dQ", "dK", "dV"), g, g0, o):
        check(("groups", _id(case), name), host64(a), ref, tol, positions=pos)
        check(("groups, statistics recomputed", _id(case), name), host64(a0), ref, tol, positions=pos)
    check(("groups dR_in", _id(case)), host64(g[3]), o[3] * e, tol)
    check(("groups dS_in", _id(case)), host64(g[4]), o[4] * e, tol)
    if feat == "favor":
        check(("groups dW", _id(case)), host64(g[5]), o[5], tol if dt == "f32" else 5e-2)


def test_groups_in_several_windows():
    # 12 slices of 100 in groups of 2, windows given as 5 slices -> 2 groups each: 3 windows
    B, H, L, d, M, C, G = 1, 2, 1200, 64, 64, 12, 2
    x = inputs(B, H, L, d, M, torch.float32, "favor", seed=93)
    dsc = A.make_desc(x["q"], M, "favor", C, window_chunks=5, group_slices=G)
    assert _lib.lib().slim_window_chunks(ctypes.byref(dsc)) == 4
    print("groups in several windows", flush=True)
    Y, R, S, rs, st = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", C, window_chunks=5, want_row_stats=True,
                                 want_states=True, group_slices=G)
    assert st is None  # several windows: nothing to keep
    g = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", C, window_chunks=5, Y=Y, row_stats=rs,
                   group_slices=G)
    torch.cuda.synchronize()
    h = {n: host64(x[n]) for n in ("q", "k", "v", "dy")}
    Yo, _, Ro, So = oracle.attn_fwd(h["q"], h["k"], h["v"], host64(x["W"]), "favor", form="prefix")
    o = oracle.attn_bwd(h["q"], h["k"], h["v"], host64(x["W"]), h["dy"], "favor", form="prefix")
    pos = (200, tile_rows(x["q"], M, "favor", C))
    check("groups/windows Y", host64(Y), Yo, 1e-4, positions=pos)
    check("groups/windows R", host64(R), Ro, 1e-4)
    for name, a, ref in zip(("dQ", "dK", "dV"), g, o):
        check(("groups/windows", name), host64(a), ref, 1e-4, positions=pos)


def test_automatic_grouping_matches_one_slice_per_workgroup():
    # 64 heads in 32 slices of 256 (M = 256): the automatic choice walks 4 slices per
    # workgroup (groups of 1024 rows, 512 workgroups: one round of the chip); against one
    # slice per workgroup
    B, H, L, d, M, C = 4, 16, 8192, 64, 256, 32
    x = inputs(B, H, L, d, M, torch.bfloat16, "favor", seed=94)
    dsc = A.make_desc(x["q"], M, "favor", C)
    assert _lib.lib().slim_group_slices(ctypes.byref(dsc)) == 4
    print("automatic grouping", flush=True)
    outs = []
    for G in (0, 1):
        Y, R, S, rs, st = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", C, want_row_stats=True,
                                     want_states=True, group_slices=G)
        g = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", C, Y=Y, row_stats=rs, states=st,
                       group_slices=G)
        outs.append((Y, R, S) + tuple(g[:3]))
    torch.cuda.synchronize()
    for name, a, b in zip(("Y", "R", "S", "dQ", "dK", "dV"), *outs):
        check(("automatic vs one slice per workgroup", name), host64(a), host64(b), 2e-2)
    # and two sampled heads against the oracle
    sel = [(0, 0), (B - 1, H - 1)]
    h = {n: np.stack([host64(x[n][b, hh]) for b, hh in sel])[None] for n in ("q", "k", "v", "dy")}
    Yo, _, _, _ = oracle.attn_fwd(h["q"], h["k"], h["v"], host64(x["W"]), "favor", form="prefix")
    o = oracle.attn_bwd(h["q"], h["k"], h["v"], host64(x["W"]), h["dy"], "favor", form="prefix")
    for name, a, ref in zip(("Y", "dQ", "dK", "dV"), (outs[0][0],) + outs[0][3:], (Yo,) + o[:3]):
        got = np.stack([host64(a[b, hh]) for b, hh in sel])[None]
        check(("automatic grouping vs oracle", name), got, ref, 2e-2, positions=(1024, tile_rows(x["q"], M, "favor", C)))  # noqa: E501
