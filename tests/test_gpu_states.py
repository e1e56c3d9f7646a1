"""The forward's per-slice states handed to the backward (include/slim.h,
slim_state_bytes; page "Sub-Linear Memory: How to Make Performers SLiM",
Subsection 3.2: the slices' entry states are the prefix sums of eq. (14)-(15) at
the slice boundaries).

  * the states the forward fills are those prefix sums: entry n of a head is
    (R, S) after the first n slices (times exp(-koff)), against the oracle's
    prefix form run on the first n*c rows;
  * a backward given them returns, bit for bit, what the backward that rebuilds
    them returns (they are the same values: same kernels, same inputs), for
    dQ, dK, dV, the state gradients and dW; so does the autograd function with
    and without kept states;
  * where the slices span several windows no states are kept and the backward
    rebuilds them as before."""
import numpy as np
import pytest
import torch

import oracle
from causal_linear_attention_amd import attention as A
from gpu_util import DT, TOL, check, gpu_koff, host64, inputs

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, L, d, M, C, dtype, feat
    (2, 3, 1000, 64, 128, 3, "f32", "favor"),     # ragged last slice
    (1, 2, 2048, 64, 256, 4, "bf16", "favor"),
    (1, 2, 1536, 128, 128, 6, "bf16", "elu1"),
    (2, 2, 700, 32, 32, 7, "f32", "elu1"),
]


def _ids(c):
    return "B%dH%dL%dd%dM%dC%d-%s-%s" % c


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_states_are_the_slice_boundary_prefix_sums(case):
    B, H, L, d, M, C, dt, feat = case
    dtype = DT[dt]
    x = inputs(B, H, L, d, M, dtype, feat, seed=81)
    print("states", _ids(case), flush=True)
    Y, R, S, rs, st = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], feat, C, want_row_stats=True, want_states=True)
    torch.cuda.synchronize()
    c = -(-L // C)
    n = -(-L // c)
    assert st is not None and tuple(st.shape) == (B, H, n + 1, d + 1, M)
    e = np.exp(gpu_koff(x["W"])) if feat == "favor" else 1.0
    h = {k: host64(x[k]) for k in ("q", "k", "v")}
    Wh = host64(x["W"]) if feat == "favor" else None
    got = host64(st) * e
    # entry 0 is the (zero) initial state; the last entry is the final state R_out, S_out
    assert np.all(got[:, :, 0] == 0.0)
    assert torch.equal(st[:, :, n, :d, :], R) and torch.equal(st[:, :, n, d, :], S)
    # fp32 sums of the features; with bf16 inputs the products take g(K) rounded to bf16
    # (2^-9 relative per term): 1.8e-3 measured on the first slice
    tol = 1e-5 if dt == "f32" else 5e-3
    for j in sorted({1, n // 2, n - 1, n}):
        rows = min(j * c, L)
        _, _, Ro, So = oracle.attn_fwd(h["q"][:, :, :rows], h["k"][:, :, :rows], h["v"][:, :, :rows], Wh, feat,
                                       form="prefix")
        check(("states R", _ids(case), j), got[:, :, j, :d, :], Ro, tol, rows_axis=False)
        check(("states S", _ids(case), j), got[:, :, j, d, :], So, tol, rows_axis=False)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_backward_with_kept_states_is_bitwise_the_rebuilding_one(case):
    B, H, L, d, M, C, dt, feat = case
    dtype = DT[dt]
    x = inputs(B, H, L, d, M, dtype, feat, seed=82)
    rng = np.random.default_rng(83)
    R0 = torch.from_numpy(rng.random((B, H, d, M)).astype(np.float32)).cuda()
    S0 = torch.from_numpy(rng.random((B, H, M)).astype(np.float32)).cuda()
    dR = torch.from_numpy(rng.standard_normal((B, H, d, M)).astype(np.float32)).cuda()
    dS = torch.from_numpy(rng.standard_normal((B, H, M)).astype(np.float32)).cuda()
    print("kept states", _ids(case), flush=True)
    q, k, v, W, dy = x["q"], x["k"], x["v"], x["W"], x["dy"]
    Y, R, S, rs, st = A.attn_fwd(q, k, v, W, feat, C, R_in=R0, S_in=S0, want_row_stats=True, want_states=True)
    Y1, R1, S1, rs1 = A.attn_fwd(q, k, v, W, feat, C, R_in=R0, S_in=S0, want_row_stats=True)
    torch.cuda.synchronize()
    assert st is not None
    for a, b in ((Y, Y1), (R, R1), (S, S1), (rs, rs1)):
        assert torch.equal(a, b)
    # the initial state is entry 0 of every head
    assert torch.equal(st[:, :, 0, :d, :], R0) and torch.equal(st[:, :, 0, d, :], S0)
    kw = dict(R_in=R0, S_in=S0, dR_out=dR, dS_out=dS, want_state_grad=True, want_dw=feat == "favor")
    for stats in ((Y, rs), (None, None)):
        with_st = A.attn_bwd(q, k, v, W, dy, feat, C, Y=stats[0], row_stats=stats[1], states=st, **kw)
        without = A.attn_bwd(q, k, v, W, dy, feat, C, Y=stats[0], row_stats=stats[1], **kw)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV", "dR_in", "dS_in", "dW"), with_st, without):
            assert torch.equal(a, b), (name, stats[0] is None)
    # and the results are the oracle's
    h = {n: host64(x[n]) for n in ("q", "k", "v", "dy")}
    Wh = host64(W) if feat == "favor" else None
    o = oracle.attn_bwd(h["q"], h["k"], h["v"], Wh, h["dy"], feat, R0=host64(R0), S0=host64(S0),
                        dRout=host64(dR), dSout=host64(dS), form="prefix")
    tol = TOL[dtype]
    for name, a, ref in zip(("dQ", "dK", "dV"), with_st, o):
        check(("kept states", _ids(case), name), host64(a), ref, tol)


def test_several_windows_keep_no_states():
    B, H, L, d, M, C = 1, 2, 4096, 64, 64, 8
    x = inputs(B, H, L, d, M, torch.bfloat16, "favor", seed=84)
    print("several windows", flush=True)
    out = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", C, window_chunks=3, want_row_stats=True,
                     want_states=True)
    assert out[4] is None
    g = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", C, window_chunks=3, Y=out[0],
                   row_stats=out[3], states=None)
    g1 = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", C, Y=out[0], row_stats=out[3])
    torch.cuda.synchronize()
    for a, b in zip(g[:3], g1[:3]):
        check("several windows vs one", host64(a), host64(b), 2e-2)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_autograd_keeps_states_with_the_same_gradients(dt):
    B, H, L, d, M, C = 2, 2, 1024, 64, 128, 4
    dtype = DT[dt]
    x = inputs(B, H, L, d, M, dtype, "favor", seed=85)
    print("autograd kept states", dt, flush=True)
    grads = []
    for keep in (True, False):
        q, k, v = (x[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
        W = x["W"].clone().requires_grad_(True)
        Y = A.slim_attention(q, k, v, W, "favor", C, keep_states=keep)
        Y.backward(x["dy"])
        torch.cuda.synchronize()
        grads.append((Y.detach(), q.grad, k.grad, v.grad, W.grad))
    for a, b in zip(*grads):
        assert torch.equal(a, b)
