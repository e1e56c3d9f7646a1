"""The projection gradient dW (slim_attn_bwd with dW) against the fp64 oracle.

g(x)_m = exp(w_m.x - |x|^2/2)/sqrt(M) (page "Sub-Linear Memory: How to Make
Performers SLiM", Subsection 2.1) depends on W only through w_m, so dW sums
(dL/dg_m) g_m x over every query and key row of every head.  The oracle's dW is
pinned by finite differences and by the rotation invariance of FAVOR+; the same
invariance is checked here on the GPU at the full headline size, where the
oracle cannot evaluate every head:  W^T dW + sum over rows of (Q^T dQ + K^T dK)
is symmetric.  Tolerance: normwise relative error of the [M, d] matrix, 1e-4
for fp32 inputs and 2e-2 for bf16 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from causal_linear_attention_amd import attention as A
from causal_linear_attention_amd import synth
from causal_linear_attention_amd.workloads import WORKLOADS
from gpu_util import DT, TOL, check, host64, inputs, relerr_heads, tile_rows

pytestmark = pytest.mark.gpu

# (B, H, L, d, M, slices, window, dtype): several tiles per slice, ragged tails,
# one slice, one-row slices, several windows (the partial sums of later windows
# are added to dW), every d and both dtypes.
CASES = [
    (1, 1, 256, 16, 16, 4, 0, "f32"),
    (1, 2, 200, 16, 32, 3, 0, "f32"),     # slice 67: ragged tiles, ragged last slice
    (2, 2, 160, 32, 64, 1, 0, "f32"),     # one slice
    (1, 2, 96, 64, 128, 96, 0, "f32"),    # one-row slices
    (1, 2, 333, 64, 256, 5, 2, "f32"),    # three windows
    (1, 1, 150, 128, 64, 3, 0, "f32"),
    (1, 2, 300, 64, 64, 7, 3, "bf16"),    # three windows
    (1, 2, 257, 64, 256, 2, 0, "bf16"),
    (2, 1, 190, 64, 128, 4, 0, "bf16"),
    (1, 2, 200, 128, 256, 3, 0, "bf16"),  # 16-row tiles
    (3, 2, 130, 32, 32, 5, 1, "bf16"),    # one slice per window
]


def _id(c):
    return "B%dH%dL%d_d%dM%d_C%d_P%d_%s" % c


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_dw_matches_oracle(case):
    B, H, L, d, M, C, P, dt = case
    dtype = DT[dt]
    print("dw", _id(case), flush=True)
    x = inputs(B, H, L, d, M, dtype, "favor", seed=51)
    q, k, v, W, dy = x["q"], x["k"], x["v"], x["W"], x["dy"]
    g = A.attn_bwd(q, k, v, W, dy, "favor", C, window_chunks=P, want_dw=True)
    plain = A.attn_bwd(q, k, v, W, dy, "favor", C, window_chunks=P)
    torch.cuda.synchronize()
    o = oracle.attn_bwd(host64(q), host64(k), host64(v), host64(W), host64(dy), "favor", want_dw=True)
    tol = TOL[dtype]
    assert g[5].shape == (M, d) and g[5].dtype == torch.float32
    check(("dW", case), host64(g[5]), o[5], tol)
    pos = (-(-L // C), tile_rows(q, M, "favor", C))
    for i, name in enumerate(("dQ", "dK", "dV")):
        check((name, case), host64(g[i]), o[i], tol, positions=pos)
        # the dW pass computes dQ, dK, dV as the plain backward does (its kernels are
        # compiled separately, so the rounding may differ in the last place)
        e = relerr_heads(host64(g[i]), host64(plain[i]))
        print(name, "dW pass vs plain backward", e)
        assert e < (1e-6 if dt == "f32" else 1e-3), name


def test_dw_with_initial_state_and_state_gradients():
    # a later piece of a streamed sequence: nonzero entry state and incoming state gradient
    B, H, L, d, M = 1, 2, 160, 64, 128
    x = inputs(B, H, L, d, M, torch.float32, "favor", seed=52)
    rng = np.random.default_rng(53)
    R0 = torch.from_numpy(rng.standard_normal((B, H, d, M)).astype(np.float32) * 0.2).cuda()
    S0 = torch.from_numpy(np.abs(rng.standard_normal((B, H, M))).astype(np.float32) + 0.5).cuda()
    dRo = torch.from_numpy(rng.standard_normal((B, H, d, M)).astype(np.float32) * 1e-2).cuda()
    dSo = torch.from_numpy(rng.standard_normal((B, H, M)).astype(np.float32) * 1e-2).cuda()
    g = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", 3, R_in=R0, S_in=S0, dR_out=dRo, dS_out=dSo,
                   want_state_grad=True, want_dw=True)
    torch.cuda.synchronize()
    o = oracle.attn_bwd(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(x["W"]), host64(x["dy"]), "favor",
                        R0=host64(R0), S0=host64(S0), dRout=host64(dRo), dSout=host64(dSo), want_dw=True)
    check("dW with state", host64(g[5]), o[5], 1e-4)
    check("dR0 with dW", host64(g[3]), o[3], 1e-4)
    check("dS0 with dW", host64(g[4]), o[4], 1e-4)


def test_dw_deterministic_and_overwritten():
    x = inputs(2, 3, 300, 64, 256, torch.bfloat16, "favor", seed=54)
    a = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", 4, window_chunks=2, want_dw=True)[5]
    b = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", 4, window_chunks=2, want_dw=True)[5]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_dw_autograd():
    # slim_attention returns W's gradient when W requires one
    x = inputs(1, 2, 130, 32, 64, torch.float32, "favor", seed=55)
    W = x["W"].clone().requires_grad_(True)
    q = x["q"].clone().requires_grad_(True)
    Y = A.slim_attention(q, x["k"], x["v"], W, "favor", 3)
    (Y * x["dy"]).sum().backward()
    torch.cuda.synchronize()
    o = oracle.attn_bwd(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(x["W"]), host64(x["dy"]), "favor",
                        want_dw=True)
    assert W.grad is not None and W.grad.dtype == W.dtype
    check("autograd dW", host64(W.grad), o[5], 1e-4)
    check("autograd dQ", host64(q.grad), o[0], 1e-4)


def _make(w):
    dt = DT[w.dtype]
    shp = (w.B, w.H, w.L, w.d)
    x = {n: synth.device_normal(w.seed, tid, shp, s).to(dt)
         for n, tid, s in (("q", synth.TID_Q, w.qkv_scale), ("k", synth.TID_K, w.qkv_scale),
                           ("v", synth.TID_V, 1.0), ("dy", synth.TID_DY, 1.0))}
    x["W"] = torch.from_numpy(synth.projection(w.seed, w.M, w.d, w.w_kind)).to(dt).cuda()
    return x


def test_dw_fullsize_rotation_symmetry_and_sampled_heads():
    # the headline workload (B=4, H=16, L=16384, d=64, M=256, bf16, 32 slices), in the
    # launch configuration the bench times, with dW
    w = WORKLOADS["favor_bf16_L16384_d64_M256"]
    print("dw fullsize", w.name, flush=True)
    x = _make(w)
    dQ, dK, _, _, _, dW = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", w.chunks, want_dw=True)
    torch.cuda.synchronize()
    assert torch.isfinite(dW).all()
    # rotation invariance: W^T dW + sum (Q^T dQ + K^T dK) is symmetric
    Wd = x["W"].double()
    Tw = Wd.t() @ dW.double()
    Tx = torch.zeros_like(Tw)
    for X, dX in ((x["q"], dQ), (x["k"], dK)):
        Xf = X.double().reshape(-1, w.d)
        Tx += Xf.t() @ dX.double().reshape(-1, w.d)
    # the antisymmetric parts of the two terms are large (about ||Tw||) and must cancel
    T = Tw + Tx
    asym, asym_w = float(torch.linalg.norm(T - T.t())), float(torch.linalg.norm(Tw - Tw.t()))
    assert asym < TOL[torch.bfloat16] * asym_w, (asym, asym_w)
    # two full-length heads against the oracle (its prefix form), through the same path
    sel = x["q"][:1, :2].contiguous(), x["k"][:1, :2].contiguous(), x["v"][:1, :2].contiguous()
    dys = x["dy"][:1, :2].contiguous()
    dW2 = A.attn_bwd(*sel, x["W"], dys, "favor", w.chunks, want_dw=True)[5]
    torch.cuda.synchronize()
    o = oracle.attn_bwd(*(host64(t) for t in sel), host64(x["W"]), host64(dys), "favor", form="prefix",
                        want_dw=True)
    check("fullsize dW", host64(dW2), o[5], TOL[torch.bfloat16])


# bf16 FAVOR+ shapes for every way the dQ and dK kernels split their W^T products over
# waves when the waves share dg(X) . g(X): one wave for several value blocks (d = 64 with
# M = 16 or 32; d = 32, M = 16), as many waves as value blocks (d = 32, M = 64; d = 16,
# M = 16), more waves than value blocks (d = 16, M = 64), and the 64-feature shape of the
# long-sequence workload; ragged tiles and slices.
SHARED_SHAPES = [(16, 16), (16, 64), (32, 16), (32, 64), (64, 16), (64, 32), (64, 64)]


@pytest.mark.parametrize("d,M", SHARED_SHAPES, ids=lambda v: str(v))
def test_shared_operand_products_all_wave_splits(d, M):
    B, H, L, C = 1, 2, 173, 3
    print("shared", d, M, flush=True)
    x = inputs(B, H, L, d, M, torch.bfloat16, "favor", seed=56)
    g = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", C, want_dw=True)
    p = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", C)
    torch.cuda.synchronize()
    o = oracle.attn_bwd(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(x["W"]), host64(x["dy"]), "favor",
                        want_dw=True)
    tol = TOL[torch.bfloat16]
    pos = (-(-L // C), tile_rows(x["q"], M, "favor", C))
    for i, name in enumerate(("dQ", "dK", "dV")):
        check(("shared", d, M, name, "dW pass"), host64(g[i]), o[i], tol, positions=pos)
        check(("shared", d, M, name), host64(p[i]), o[i], tol, positions=pos)
    check(("shared", d, M, "dW"), host64(g[5]), o[5], tol)
