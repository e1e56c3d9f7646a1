"""The key-side offset of W (include/slim.h, "Key-side offset"): FAVOR+ with rows of W
of large norm and keys placed on top of them, where exp(w_m.k - |k|^2/2) exceeds the
fp32 range (page "Sub-Linear Memory: How to Make Performers SLiM", Subsection 2.1:
positive features make the division well defined and stable; that needs them
finite).

Every call scales the key features by exp(-koff), koff = max(0, max_m |w_m|^2/2 - 60),
which cancels in Y, dQ, dK, dV: those are compared with the fp64 oracle (which needs
no offset: fp64 holds exp(120)) at the usual bounds; the states that cross the
boundary are compared after multiplying by exp(koff), and the state gradients after
the matching change of variables."""
import numpy as np
import pytest
import torch

import oracle
from causal_linear_attention_amd import attention as A
from causal_linear_attention_amd import synth
from gpu_util import DT, TOL, check, gpu_koff, host64, koff_of, tile_rows, to_dev

pytestmark = pytest.mark.gpu

B, H, L, d, M, C = 1, 2, 700, 64, 64, 3
BIG = {5: 200.0, 20: 220.0, 41: 240.0}  # W row -> |w|^2 (koff = 240/2 - 60 = 60)
NEAR = {137: 5, 300: 41, 411: 20, 650: 41, 233: 5, 234: 20}  # key row -> the W row it sits on


def _inputs(dtype, seed=61):
    Wn = synth.projection(seed, M, d, "gaussian").astype(np.float64)
    for m, n2 in BIG.items():
        Wn[m] *= np.sqrt(n2 / np.sum(Wn[m] ** 2))
    W = to_dev(Wn, dtype)
    sc = d ** -0.25
    q = synth.normal(seed, synth.TID_Q, B, H, L, d, sc)
    k = synth.normal(seed, synth.TID_K, B, H, L, d, sc)
    noise = synth.normal(seed + 1, synth.TID_K, B, H, L, d, 0.05)
    Wr = host64(W)
    for row, m in NEAR.items():
        k[:, :, row] = Wr[m] + noise[:, :, row]
    x = dict(q=to_dev(q, dtype), k=to_dev(k, dtype), W=W,
             v=to_dev(synth.normal(seed, synth.TID_V, B, H, L, d, 1.0), dtype),
             dy=to_dev(synth.normal(seed, synth.TID_DY, B, H, L, d, 1.0), dtype))
    return x


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_large_norm_projection_rows(dt):
    dtype = DT[dt]
    tol = TOL[dtype]
    x = _inputs(dtype)
    q, k, v, W, dy = x["q"], x["k"], x["v"], x["W"], x["dy"]
    h = {n: host64(x[n]) for n in ("q", "k", "v", "W", "dy")}
    # without an offset these keys' features overflow fp32 (exp(88.7) is its largest value)
    expo = h["k"] @ h["W"].T - 0.5 * np.sum(h["k"] ** 2, axis=-1, keepdims=True)
    assert float(expo.max()) > 100.0, float(expo.max())
    print("largest key exponent %.1f, koff %.2f" % (float(expo.max()), koff_of(W)), flush=True)

    ko = torch.full((1,), -1.0, device="cuda")
    Y, R, S, rs = A.attn_fwd(q, k, v, W, "favor", C, want_row_stats=True, koff_out=ko)
    g = A.attn_bwd(q, k, v, W, dy, "favor", C, Y=Y, row_stats=rs, want_dw=True)
    g0 = A.attn_bwd(q, k, v, W, dy, "favor", C)  # the backward that recomputes the statistics
    torch.cuda.synchronize()
    kf = float(ko)
    assert abs(kf - koff_of(W)) <= 1e-5 * kf and kf > 50.0, (kf, koff_of(W))
    for t in (Y, R, S, *g, *g0[:3]):
        if t is not None:
            assert torch.isfinite(t).all()

    Yo, den, Ro, So = oracle.attn_fwd(h["q"], h["k"], h["v"], h["W"], "favor")
    o = oracle.attn_bwd(h["q"], h["k"], h["v"], h["W"], h["dy"], "favor", want_dw=True)
    pos = (-(-L // C), tile_rows(q, M, "favor", C))
    check(("koff Y", dt), host64(Y), Yo, tol, positions=pos)
    check(("koff R", dt), host64(R) * np.exp(kf), Ro, tol)
    check(("koff S", dt), host64(S) * np.exp(kf), So, tol)
    # dQ in bf16: after each key placed on a large row of W, that one key carries nearly
    # all of a row's weight, so dQ_t (whose terms sum to zero over the keys, weighted by
    # P[t][s]) is the difference of nearly equal terms, each rounded to bf16 as an MFMA
    # operand; measured 2.6e-2 normwise here, against 5e-3 on ordinary inputs.  dW is
    # built from the same dg(Q) . g(Q) and dg(K) . g(K) rows: 3.7e-2 here
    dq_tol = 5e-2 if dt == "bf16" else tol
    for i, nm in enumerate(("dQ", "dK", "dV")):
        check(("koff", dt, nm), host64(g[i]), o[i], dq_tol if nm == "dQ" else tol, positions=pos)
        check(("koff recomputed statistics", dt, nm), host64(g0[i]), o[i], dq_tol if nm == "dQ" else tol,
              positions=pos)
    check(("koff dW", dt), host64(g[5]), o[5], dq_tol)
    # the row statistics give the denominators with the offset put back.  The features of
    # the keys on large rows have exponents built from terms near |w_m|^2 = 240, whose fp32
    # rounding is relative error of about 1e-5 in those features, and they dominate the
    # denominators they enter: 1e-4 here, against 1e-5 for ordinary fp32 inputs
    r = host64(rs)
    got = np.exp(kf - r[..., 1] * np.log(2.0) - 0.5 * np.sum(h["q"] ** 2, axis=-1)) / (r[..., 0] * np.sqrt(M))
    check(("koff denominators", dt), got[..., None], den[..., None], 1e-4 if dt == "f32" else 1e-2)


def test_scaled_states_stream_between_calls():
    # a sequence streamed through two calls with the same W: the scaled state handed over
    # is read back with the same offset, so the pieces give the one-call result, and the
    # state gradients are those of the scaled states
    dtype = torch.float32
    x = _inputs(dtype, seed=62)
    q, k, v, W, dy = x["q"], x["k"], x["v"], x["W"], x["dy"]
    cut = 350
    Yf, Rf, Sf = A.attn_fwd(q, k, v, W, "favor", C)
    first = [t[:, :, :cut].contiguous() for t in (q, k, v)]
    second = [t[:, :, cut:].contiguous() for t in (q, k, v, dy)]
    _, R1, S1 = A.attn_fwd(*first, W, "favor", 2)
    Y2, R2, S2 = A.attn_fwd(*second[:3], W, "favor", 2, R_in=R1, S_in=S1)
    torch.cuda.synchronize()
    kf = gpu_koff(W)  # the factor the library applied (within fp32 rounding of koff_of(W))
    check("streamed Y", host64(Y2), host64(Yf[:, :, cut:]), 1e-4)
    check("streamed R", host64(R2), host64(Rf), 1e-4)
    check("streamed S", host64(S2), host64(Sf), 1e-4)
    # backward of the second piece with incoming gradients of its (scaled) final state
    rng = np.random.default_rng(63)
    dRs = torch.from_numpy(rng.standard_normal((B, H, d, M)).astype(np.float32)).cuda()
    dSs = torch.from_numpy(rng.standard_normal((B, H, M)).astype(np.float32)).cuda()
    gq, gk, gv, dR1, dS1 = A.attn_bwd(*second[:3], W, second[3], "favor", 2, R_in=R1, S_in=S1, dR_out=dRs,
                                      dS_out=dSs, want_state_grad=True)
    torch.cuda.synchronize()
    e = np.exp(kf)
    h2 = [host64(t) for t in second]
    # the oracle works with the true states: R = scaled * e^koff, and a gradient with
    # respect to the scaled state is e^koff times the gradient with respect to the true one
    o = oracle.attn_bwd(*h2[:3], host64(W), h2[3], "favor", R0=host64(R1) * e, S0=host64(S1) * e,
                        dRout=host64(dRs) / e, dSout=host64(dSs) / e)
    for nm, got, ref in (("dQ", gq, o[0]), ("dK", gk, o[1]), ("dV", gv, o[2]), ("dR_in", dR1, o[3] * e),
                         ("dS_in", dS1, o[4] * e)):
        check(("streamed backward", nm), host64(got), ref, 1e-4)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_decode_continues_the_scaled_state(dt):
    # the decode step computes the same offset from W and continues the forward's state
    dtype = DT[dt]
    x = _inputs(dtype, seed=64)
    q, k, v, W = x["q"], x["k"], x["v"], x["W"]
    _, R, S = A.attn_fwd(q[:, :, :-1].contiguous(), k[:, :, :-1].contiguous(), v[:, :, :-1].contiguous(), W,
                         "favor", C)
    tok = [t[:, :, -1, :].contiguous() for t in (q, k, v)]
    tok[1] = (W[41] + 0.01 * tok[1][0, 0]).expand(B, H, d).contiguous()  # the new key on a large row
    y, R2, S2 = A.decode_step(*tok, W, "favor", R, S)
    torch.cuda.synchronize()
    e = np.exp(gpu_koff(W))
    yo, Ro, So = oracle.decode_step(*tok, W, "favor", host64(R) * e, host64(S) * e)
    assert torch.isfinite(y).all() and torch.isfinite(R2).all()
    check(("decode after large keys y", dt), host64(y), yo, TOL[dtype])
    # the new key's feature exp(w_m.k - |k|^2/2 - koff) has an argument built from terms near
    # |w_m|^2 = 240: their fp32 rounding (about 240 * 2^-24 per term) is relative error
    # 1e-5 in the feature itself, so the state is held to 1e-4 here, not the usual 1e-5
    check(("decode after large keys R", dt), host64(R2) * e, Ro, 1e-4)
    check(("decode after large keys S", dt), host64(S2) * e, So, 1e-4)
