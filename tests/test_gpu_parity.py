"""GPU (HIP, gfx950) against the fp64 oracle, element by element on the same
seeded inputs, through the C ABI.  Bounds (gpu_util.check): normwise relative
error per (batch, head) and tensor below 1e-4 for fp32 inputs and 2e-2 for bf16
inputs, max-abs/max-ref below twice that, the worst row below ten times that.  States
cross the boundary scaled by exp(-koff) (the key-side offset of W); they are
compared with the oracle's after multiplying by exp(koff)."""
import numpy as np
import pytest
import torch

import oracle
from causal_linear_attention_amd import attention as A
from gpu_util import DT, TOL, check, gpu_koff, host64, inputs, koff_of, relerr_heads, tile_rows

pytestmark = pytest.mark.gpu

# (B, H, L, d, M, chunks, dtype, feat): several tiles per chunk, ragged tails,
# a single chunk (pure intra-chunk), one-row chunks, partial last chunk.
CASES = [
    (1, 1, 256, 16, 16, 4, "f32", "favor"),    # the small fp32 forward workload
    (1, 2, 200, 16, 32, 3, "f32", "favor"),    # chunk 67: ragged tiles and ragged last chunk
    (2, 2, 160, 32, 64, 1, "f32", "favor"),    # one chunk
    (1, 2, 96, 64, 128, 96, "f32", "favor"),   # one-row chunks
    (1, 2, 333, 64, 256, 5, "f32", "favor"),
    (1, 2, 300, 64, 64, 7, "bf16", "favor"),
    (1, 2, 257, 64, 256, 2, "bf16", "favor"),
    (2, 1, 190, 64, 128, 4, "bf16", "favor"),
    (1, 2, 150, 32, 32, 3, "f32", "elu1"),
    (1, 2, 270, 64, 64, 4, "bf16", "elu1"),
    (1, 1, 200, 128, 128, 3, "bf16", "elu1"),
    (1, 1, 100, 128, 128, 2, "f32", "elu1"),
    (1, 1, 64, 16, 16, 64, "bf16", "elu1"),
    (1, 2, 200, 128, 128, 3, "bf16", "favor"),  # d = 128: the key-side offset of W is above 0
    (1, 1, 150, 128, 64, 2, "f32", "favor"),
]


def _id(c):
    return "B%dH%dL%d_d%dM%d_C%d_%s_%s" % c


def _supported(d, M, dtype, feat):
    from causal_linear_attention_amd import _lib
    import ctypes
    dsc = _lib.desc(1, 1, 16, d, M, 1, 0, _lib.SLIM_F32 if dtype == "f32" else _lib.SLIM_BF16,
                    _lib.SLIM_FEAT_FAVOR if feat == "favor" else _lib.SLIM_FEAT_ELU1)
    return _lib.lib().slim_validate(ctypes.byref(dsc), 1) == 0


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_forward_matches_oracle(case):
    B, H, L, d, M, C, dt, feat = case
    if not _supported(d, M, dt, feat):
        pytest.skip("shape not compiled")
    dtype = DT[dt]
    x = inputs(B, H, L, d, M, dtype, feat, seed=11, dy=False)
    print("fwd", _id(case), flush=True)
    ko = torch.full((1,), -1.0, device="cuda")
    Y, R, S = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], feat, C, koff_out=ko)
    torch.cuda.synchronize()
    Yo, _, Ro, So = oracle.attn_fwd(host64(x["q"]), host64(x["k"]), host64(x["v"]),
                                    None if x["W"] is None else host64(x["W"]), feat)
    tol = TOL[dtype]
    kf = float(ko)
    assert abs(kf - koff_of(x["W"])) <= 1e-5 * max(1.0, kf), (kf, koff_of(x["W"]))
    pos = (-(-L // C), tile_rows(x["q"], M, feat, C))
    check(("Y", case), host64(Y), Yo, tol, positions=pos)
    check(("R", case), host64(R) * np.exp(kf), Ro, tol)
    check(("S", case), host64(S) * np.exp(kf), So, tol)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_backward_matches_oracle(case):
    B, H, L, d, M, C, dt, feat = case
    if not _supported(d, M, dt, feat):
        pytest.skip("shape not compiled")
    dtype = DT[dt]
    x = inputs(B, H, L, d, M, dtype, feat, seed=12)
    print("bwd", _id(case), flush=True)
    Y, R, S = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], feat, C)
    dQ, dK, dV, _, _ = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], feat, C)
    torch.cuda.synchronize()
    Wh = None if x["W"] is None else host64(x["W"])
    g = oracle.attn_bwd(host64(x["q"]), host64(x["k"]), host64(x["v"]), Wh, host64(x["dy"]), feat)
    tol = TOL[dtype]
    pos = (-(-L // C), tile_rows(x["q"], M, feat, C))
    for name, got, ref in (("dQ", dQ, g[0]), ("dK", dK, g[1]), ("dV", dV, g[2])):
        check((name, case), host64(got), ref, tol, positions=pos)


@pytest.mark.parametrize("dt,feat,d,M", [("f32", "favor", 64, 128), ("bf16", "favor", 64, 256),
                                         ("bf16", "elu1", 64, 64)])
def test_featmap_matches_oracle(dt, feat, d, M):
    dtype = DT[dt]
    x = inputs(2, 3, 77, d, M, dtype, feat, seed=13, dy=False)
    phi = A.featmap(x["q"], x["W"], feat)
    Wh = None if x["W"] is None else host64(x["W"])
    ref = oracle.featmap(host64(x["q"]), Wh, feat)
    check(("featmap", dt, feat), host64(phi), ref, 1e-5 if dt == "f32" else 1e-5 * 4)
    if feat == "favor":
        phi2, off = A.featmap(x["q"], x["W"], feat, row_offset=True)
        back = host64(phi2) * np.exp(host64(off))[..., None]
        check(("featmap with row offsets", dt), back, ref, 1e-4)
        assert float(host64(phi2).max()) <= 1.0 / np.sqrt(M) * (1 + 1e-5)


def test_initial_state_and_state_gradients():
    # Streaming: run [P; X] in one call vs X from the state of P; gradients of the
    # initial state against the oracle with a nonzero incoming state gradient.
    B, H, L, d, M = 1, 2, 192, 64, 128
    dtype = torch.float32
    x = inputs(B, H, L, d, M, dtype, "favor", seed=14)
    q, k, v, W, dy = x["q"], x["k"], x["v"], x["W"], x["dy"]
    Yf, Rf, Sf = A.attn_fwd(q, k, v, W, "favor", 3)
    _, Rp, Sp = A.attn_fwd(q[:, :, :64].contiguous(), k[:, :, :64].contiguous(), v[:, :, :64].contiguous(), W,
                           "favor", 2)
    Y2, R2, S2 = A.attn_fwd(q[:, :, 64:].contiguous(), k[:, :, 64:].contiguous(), v[:, :, 64:].contiguous(), W,
                            "favor", 2, R_in=Rp, S_in=Sp)
    torch.cuda.synchronize()
    assert relerr_heads(host64(Y2), host64(Yf[:, :, 64:])) < 1e-5
    assert relerr_heads(host64(R2), host64(Rf)) < 1e-5
    rng = np.random.default_rng(5)
    dRo = torch.from_numpy(rng.standard_normal((B, H, d, M)).astype(np.float32)).cuda() * 1e-3
    dSo = torch.from_numpy(rng.standard_normal((B, H, M)).astype(np.float32)).cuda() * 1e-3
    qs, ks, vs, dys = (t[:, :, 64:].contiguous() for t in (q, k, v, dy))
    dQ, dK, dV, dR0, dS0 = A.attn_bwd(qs, ks, vs, W, dys, "favor", 2, R_in=Rp, S_in=Sp, dR_out=dRo,
                                      dS_out=dSo, want_state_grad=True)
    torch.cuda.synchronize()
    g = oracle.attn_bwd(host64(qs), host64(ks), host64(vs), host64(W), host64(dys), "favor", R0=host64(Rp),
                        S0=host64(Sp), dRout=host64(dRo), dSout=host64(dSo))
    for name, got, ref in (("dQ", dQ, g[0]), ("dK", dK, g[1]), ("dV", dV, g[2]), ("dR0", dR0, g[3]),
                           ("dS0", dS0, g[4])):
        check(("state gradients", name), host64(got), ref, 1e-4)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fp64_states(dt):
    # States passed between calls in fp64 (desc.state_dtype = SLIM_F64): streaming a
    # sequence in three pieces gives the one-call result to within the internal
    # rounding (no fp32 rounding of the states between calls), and every state and
    # state gradient matches the oracle.
    B, H, L, d, M = 1, 2, 192, 64, 128
    x = inputs(B, H, L, d, M, DT[dt], "favor", seed=15)
    q, k, v, W, dy = x["q"], x["k"], x["v"], x["W"], x["dy"]
    Yf, Rf, Sf = A.attn_fwd(q, k, v, W, "favor", 3, state_dtype=torch.float64)
    assert Rf.dtype == torch.float64 and Sf.dtype == torch.float64
    R = S = None
    ys = []
    for a, b in ((0, 48), (48, 112), (112, 192)):
        sl = [t[:, :, a:b].contiguous() for t in (q, k, v)]
        y, R, S = A.attn_fwd(*sl, W, "favor", 1, R_in=R, S_in=S, state_dtype=torch.float64)
        ys.append(y)
    torch.cuda.synchronize()
    assert relerr_heads(host64(R), host64(Rf)) < 1e-12 + 1e-6
    assert relerr_heads(host64(torch.cat(ys, 2)), host64(Yf)) < (1e-5 if dt == "f32" else 1e-2)
    Yo, _, Ro, So = oracle.attn_fwd(host64(q), host64(k), host64(v), host64(W), "favor", form="prefix")
    check(("fp64 states R", dt), host64(Rf), Ro, 1e-5 if dt == "f32" else 2e-2)
    check(("fp64 states S", dt), host64(Sf), So, 1e-5 if dt == "f32" else 2e-2)
    # backward of the last piece from its fp64 entry state, with an fp64 incoming state gradient
    rng = np.random.default_rng(6)
    dRo = torch.from_numpy(rng.standard_normal((B, H, d, M)) * 1e-3).cuda()
    dSo = torch.from_numpy(rng.standard_normal((B, H, M)) * 1e-3).cuda()
    _, Rp, Sp = A.attn_fwd(q[:, :, :112].contiguous(), k[:, :, :112].contiguous(), v[:, :, :112].contiguous(), W,
                           "favor", 2, state_dtype=torch.float64)
    qs, ks, vs, dys = (t[:, :, 112:].contiguous() for t in (q, k, v, dy))
    dQ, dK, dV, dR0, dS0 = A.attn_bwd(qs, ks, vs, W, dys, "favor", 2, R_in=Rp, S_in=Sp, dR_out=dRo,
                                      dS_out=dSo, want_state_grad=True)
    torch.cuda.synchronize()
    assert dR0.dtype == torch.float64
    g = oracle.attn_bwd(host64(qs), host64(ks), host64(vs), host64(W), host64(dys), "favor", R0=host64(Rp),
                        S0=host64(Sp), dRout=host64(dRo), dSout=host64(dSo))
    tol = TOL[DT[dt]]
    for name, got, ref in (("dQ", dQ, g[0]), ("dK", dK, g[1]), ("dV", dV, g[2]), ("dR0", dR0, g[3]),
                           ("dS0", dS0, g[4])):
        check(("fp64 states", dt, name), host64(got), ref, tol)


@pytest.mark.parametrize("window", [0, 4])
def test_backward_wide_dynamic_range(window):
    # fp32 keys scaled up so that g(K) spans many orders of magnitude: the final
    # state is dominated by a few rows and every earlier entry state is tiny next
    # to it.  Entry states rebuilt forward with fp64 carries keep 1e-4; recovering
    # them from the fp32 final state by subtraction does not (regression case).
    B, H, L, d, M, C = 1, 2, 2048, 64, 128, 16
    x = inputs(B, H, L, d, M, torch.float32, "favor", seed=21, w_kind="orthogonal")
    x["k"] = x["k"] * 1.6
    print("wide range, window", window, flush=True)
    Y, R, S = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", C, window_chunks=window)
    dQ, dK, dV, _, _ = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", C, window_chunks=window)
    torch.cuda.synchronize()
    h = [host64(x[n]) for n in ("q", "k", "v")]
    g = oracle.attn_bwd(*h, host64(x["W"]), host64(x["dy"]), "favor", form="prefix")
    for name, got, ref in (("dQ", dQ, g[0]), ("dK", dK, g[1]), ("dV", dV, g[2])):
        check(("wide range", window, name), host64(got), ref, 1e-4)


def test_chunk_count_invariance_and_windows():
    # The sliced result does not depend on the slice count or the window (up to rounding).
    B, H, L, d, M = 1, 2, 1024, 64, 64
    x = inputs(B, H, L, d, M, torch.float32, "favor", seed=15)
    ref = None
    for C, P in ((1, 0), (4, 0), (16, 0), (16, 3), (64, 5), (1024, 100)):
        Y, R, S = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", C, window_chunks=P)
        dQ, dK, dV, _, _ = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", C, window_chunks=P)
        cur = [host64(t) for t in (Y, dQ, dK, dV)]
        if ref is None:
            ref = cur
            g = oracle.attn_bwd(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(x["W"]), host64(x["dy"]),
                                "favor")
            Yo = oracle.attn_fwd(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(x["W"]), "favor")[0]
            oref = [Yo, g[0], g[1], g[2]]
        errs = [relerr_heads(a, b) for a, b in zip(cur, ref)]
        oerrs = [relerr_heads(a, b) for a, b in zip(cur, oref)]
        print("slices", C, "window", P, "vs one slice", ["%.2e" % e for e in errs],
              "vs oracle", ["%.2e" % e for e in oerrs], flush=True)
        # each chunking matches the oracle, hence the others, within the fp32 bound
        pos = (-(-L // C), tile_rows(x["q"], M, "favor", C))
        for nm, a, b in zip(("Y", "dQ", "dK", "dV"), cur, oref):
            check(("slices", C, "window", P, nm), a, b, 1e-4, positions=pos)
        assert max(errs) < 2e-4, (C, P, errs)


def test_deterministic():
    x = inputs(1, 2, 700, 64, 256, torch.bfloat16, "favor", seed=16)
    outs = []
    for _ in range(2):
        Y, R, S = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", 3)
        dQ, dK, dV, _, _ = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", 3)
        outs.append([t.clone() for t in (Y, R, dQ, dK, dV)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_causality():
    # Perturbing row j leaves outputs before j bitwise unchanged.
    x = inputs(1, 1, 256, 64, 64, torch.float32, "favor", seed=17, dy=False)
    Y0, _, _ = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", 4)
    for name in ("q", "k", "v"):
        y = dict(x)
        t = x[name].clone()
        t[:, :, 150] += 0.5
        y[name] = t
        Y1, _, _ = A.attn_fwd(y["q"], y["k"], y["v"], y["W"], "favor", 4)
        torch.cuda.synchronize()
        assert torch.equal(Y0[:, :, :150], Y1[:, :, :150]), name
        assert not torch.equal(Y0[:, :, 150], Y1[:, :, 150]), name


def test_autograd_function():
    x = inputs(1, 2, 130, 32, 64, torch.float32, "favor", seed=18)
    q, k, v = (x[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    Y = A.slim_attention(q, k, v, x["W"], "favor", 3)
    (Y * x["dy"]).sum().backward()
    g = oracle.attn_bwd(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(x["W"]), host64(x["dy"]), "favor")
    for nm, got, ref in (("dQ", q.grad, g[0]), ("dK", k.grad, g[1]), ("dV", v.grad, g[2])):
        check(("autograd", nm), host64(got), ref, 1e-4)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_forward_row_stats_give_the_denominators(case):
    # row_stats = (1/den', o) with den = den' 2^-o exp(-|q|^2/2) / sqrt(M) (FAVOR+), den = den' (elu+1)
    B, H, L, d, M, C, dt, feat = case
    if not _supported(d, M, dt, feat):
        pytest.skip("shape not compiled")
    dtype = DT[dt]
    x = inputs(B, H, L, d, M, dtype, feat, seed=15, dy=False)
    Y, R, S, rs = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], feat, C, want_row_stats=True)
    Y0, _, _ = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], feat, C)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y0)  # asking for the statistics changes nothing else
    q = host64(x["q"])
    _, den, _, _ = oracle.attn_fwd(q, host64(x["k"]), host64(x["v"]), None if x["W"] is None else host64(x["W"]),
                                   feat)
    r = host64(rs)
    got = 1.0 / r[..., 0]
    if feat == "favor":
        kf = gpu_koff(x["W"])  # the factor the library applied (koff_of(W) up to fp32 rounding)
        got = got * np.exp(kf - r[..., 1] * np.log(2.0) - 0.5 * np.sum(q * q, axis=-1)) / np.sqrt(M)
    else:
        assert np.all(r[..., 1] == 0)
    check(("denominators", case), got[..., None], den[..., None], 1e-5 if dt == "f32" else 1e-2)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_backward_from_forward_row_stats_matches_oracle(case):
    # the backward that takes the forward's Y and row statistics instead of recomputing them
    B, H, L, d, M, C, dt, feat = case
    if not _supported(d, M, dt, feat):
        pytest.skip("shape not compiled")
    dtype = DT[dt]
    x = inputs(B, H, L, d, M, dtype, feat, seed=12)
    print("bwd from row stats", _id(case), flush=True)
    Y, R, S, rs = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], feat, C, want_row_stats=True)
    g = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], feat, C, Y=Y, row_stats=rs)
    g0 = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], feat, C)
    torch.cuda.synchronize()
    Wh = None if x["W"] is None else host64(x["W"])
    o = oracle.attn_bwd(host64(x["q"]), host64(x["k"]), host64(x["v"]), Wh, host64(x["dy"]), feat)
    tol = TOL[dtype]
    pos = (-(-L // C), tile_rows(x["q"], M, feat, C))
    for i, name in enumerate(("dQ", "dK", "dV")):
        e0 = relerr_heads(host64(g[i]), host64(g0[i]))
        m = check(("bwd from row stats", case, name), host64(g[i]), o[i], tol, positions=pos)
        print(name, "vs oracle", m, "vs recomputed statistics %.2e" % e0)


def test_row_stats_across_windows_and_slice_counts():
    # statistics from a forward with another slice count and window, a nonzero initial
    # state and incoming state gradients
    B, H, L, d, M = 1, 2, 300, 64, 128
    x = inputs(B, H, L, d, M, torch.float32, "favor", seed=16)
    rng = np.random.default_rng(17)
    R0 = torch.from_numpy(rng.standard_normal((B, H, d, M)).astype(np.float32) * 0.2).cuda()
    S0 = torch.from_numpy(np.abs(rng.standard_normal((B, H, M))).astype(np.float32) + 0.5).cuda()
    dRo = torch.from_numpy(rng.standard_normal((B, H, d, M)).astype(np.float32) * 1e-2).cuda()
    dSo = torch.from_numpy(rng.standard_normal((B, H, M)).astype(np.float32) * 1e-2).cuda()
    Y, _, _, rs = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", 1, R_in=R0, S_in=S0, want_row_stats=True)
    g = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", 7, R_in=R0, S_in=S0, dR_out=dRo, dS_out=dSo,
                   want_state_grad=True, window_chunks=2, Y=Y, row_stats=rs, want_dw=True)
    torch.cuda.synchronize()
    o = oracle.attn_bwd(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(x["W"]), host64(x["dy"]), "favor",
                        R0=host64(R0), S0=host64(S0), dRout=host64(dRo), dSout=host64(dSo), want_dw=True)
    for i, name in enumerate(("dQ", "dK", "dV", "dR0", "dS0")):
        check(("row stats across windows", name), host64(g[i]), o[i], 1e-4)
    check(("row stats across windows", "dW"), host64(g[5]), o[5], 1e-4)


def test_most_heads_one_launch_allows():
    # B*H = 65535 (the largest head count the chunk kernels' grid takes): forward,
    # backward from the kept row statistics and dW; sampled heads against the oracle,
    # dW (a sum over every head) against the oracle over all heads
    B, H, L, d, M, C = 65535, 1, 40, 16, 16, 2
    print("most heads", B * H, flush=True)
    x = inputs(B, H, L, d, M, torch.bfloat16, "favor", seed=19)
    Y, R, S, rs = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", C, want_row_stats=True)
    g = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", C, Y=Y, row_stats=rs, want_dw=True)
    torch.cuda.synchronize()
    h = {n: host64(x[n]) for n in ("q", "k", "v", "dy")}
    Wh = host64(x["W"])
    o = oracle.attn_bwd(h["q"], h["k"], h["v"], Wh, h["dy"], "favor", form="prefix", want_dw=True)
    idx = np.concatenate([[0, B - 1], np.random.default_rng(0).choice(B, 62, replace=False)])
    Yo = oracle.attn_fwd(h["q"][idx], h["k"][idx], h["v"][idx], Wh, "favor")[0]
    tol = TOL[torch.bfloat16]
    check(("most heads", "Y"), host64(Y)[idx], Yo, tol)
    for i, name in enumerate(("dQ", "dK", "dV")):
        check(("most heads", name), host64(g[i])[idx], o[i][idx], tol)
    check(("most heads", "dW"), host64(g[5]), o[5], tol)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("feat", ["favor", "elu1"])
def test_degenerate_closed_forms(dt, feat):
    # closed forms of eq. (2), not the oracle: a one-row sequence gives Y = V, dQ = dK = 0,
    # dV = dY; values constant along the sequence give Y = V and dQ = dK = 0, whatever
    # the slicing, with either backward ("0" up to rounding: against the size of dV)
    dtype = DT[dt]
    d = 64
    M = 128 if feat == "favor" else d
    tol = 1e-5 if dt == "f32" else TOL[dtype]
    zero = 5e-4 if dt == "f32" else 5e-2  # "vanishes": against the gradients' own size
    x = inputs(2, 3, 1, d, M, dtype, feat, seed=20)
    Y, _, _, rs = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], feat, 1, want_row_stats=True)
    for kept in (True, False):
        g = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], feat, 1, Y=Y if kept else None,
                       row_stats=rs if kept else None)
        torch.cuda.synchronize()
        check(("one row: Y = V", dt, feat), host64(Y), host64(x["v"]), tol)
        scale = float(x["dy"].abs().max())
        assert float(g[0].abs().max()) < zero * scale and float(g[1].abs().max()) < zero * scale, kept
        check(("one row: dV = dY", dt, feat, kept), host64(g[2]), host64(x["dy"]), tol)
    L = 200
    x = inputs(1, 2, L, d, M, dtype, feat, seed=21)
    v = x["v"][:, :, :1].expand(-1, -1, L, -1).contiguous()
    for C, P in ((1, 0), (7, 0), (200, 3)):
        Y, _, _, rs = A.attn_fwd(x["q"], x["k"], v, x["W"], feat, C, window_chunks=P, want_row_stats=True)
        for kept in (True, False):
            g = A.attn_bwd(x["q"], x["k"], v, x["W"], x["dy"], feat, C, window_chunks=P, Y=Y if kept else None,
                           row_stats=rs if kept else None)
            torch.cuda.synchronize()
            check(("constant V: Y = V", dt, feat, C, P), host64(Y), host64(v), tol)
            # dQ, dK vanish up to rounding: compare with the size of dV's contributions
            scale = float(g[2].abs().max())
            assert float(g[0].abs().max()) < zero * scale and float(g[1].abs().max()) < zero * scale, (C, P, kept)
