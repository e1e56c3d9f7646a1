"""Parity of the recurrent decode step (slim_decode_step) with the fp64 oracle.

The oracle's decode step is its prefix-sum recurrence run over one position
(page "Sub-Linear Memory: How to Make Performers SLiM", Subsection 2.1,
eq. (3)-(4)); it receives exactly the values the GPU received (io-dtype
inputs, the fp32 state).  Outputs y are checked at the io dtype's tolerance,
the fp32 states at 1e-5 (gpu_util.check: normwise, max-abs/max-ref, worst row).
States cross the boundary times exp(-koff), the key-side offset of W: the
oracle gets them multiplied back by exp(koff), and so are the results.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DT, TOL, check, gpu_koff, host64, inputs, relerr_heads
from causal_linear_attention_amd import attention as A

pytestmark = pytest.mark.gpu

TOL_STATE = 1e-5

# (B, H, d, M, dtype, feat)
CASES = [
    (3, 5, 64, 256, "bf16", "favor"),
    (2, 3, 16, 16, "f32", "favor"),
    (1, 7, 32, 64, "f32", "favor"),
    (2, 2, 128, 256, "bf16", "favor"),
    (2, 4, 64, 64, "bf16", "favor"),
    (1, 3, 16, 256, "f32", "favor"),
    (3, 2, 128, 128, "bf16", "elu1"),
    (2, 2, 16, 16, "f32", "elu1"),
]


def _ids(c):
    return "B%d_H%d_d%d_M%d_%s_%s" % c


def _token(B, H, d, M, dt, feat, seed, scale=None):
    t = inputs(B, H, 1, d, M, DT[dt], feat, seed=seed, scale=scale, dy=False)
    q, k, v = (t[n][:, :, 0, :].contiguous() for n in ("q", "k", "v"))
    return q, k, v, t["W"]


def _state(B, H, d, M, dt, feat, seed, W, L=12):
    """A state reached by a real prefix of L tokens (fp32 on the device), scaled by
    exp(-koff) as the library holds states."""
    t = inputs(B, H, L, d, M, DT[dt], feat, seed=seed, dy=False)
    _, _, R, S = oracle.attn_fwd(t["q"], t["k"], t["v"], W, feat, form="prefix")
    sc = np.exp(-gpu_koff(W))
    return (torch.from_numpy(R * sc).float().cuda().contiguous(), torch.from_numpy(S * sc).float().cuda().contiguous())


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_decode_step_matches_oracle(case):
    B, H, d, M, dt, feat = case
    print("decode", case, flush=True)
    q, k, v, W = _token(B, H, d, M, dt, feat, seed=31)
    R, S = _state(B, H, d, M, dt, feat, 32, W)
    y, R2, S2 = A.decode_step(q, k, v, W, feat, R, S)
    torch.cuda.synchronize()
    sc = np.exp(gpu_koff(W))
    yo, Ro, So = oracle.decode_step(q, k, v, W, feat, host64(R) * sc, host64(S) * sc)
    check(("decode y", case), host64(y), yo, TOL[DT[dt]])
    check(("decode R", case), host64(R2) * sc, Ro, TOL_STATE)
    check(("decode S", case), host64(S2) * sc, So, TOL_STATE)
    # inputs untouched (not in place)
    assert torch.equal(R, _state(B, H, d, M, dt, feat, 32, W)[0])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("feat", ["favor", "elu1"])
def test_first_token_gives_its_value(dt, feat):
    B, H, d = 2, 3, 64
    M = 128 if feat == "favor" else d
    q, k, v, W = _token(B, H, d, M, dt, feat, seed=33)
    y, R, S = A.decode_step(q, k, v, W, feat)
    torch.cuda.synchronize()
    if dt == "bf16":  # v (1 + O(1e-7)) rounds back to v
        assert torch.equal(y, v)
    else:
        check(("first token y = v", feat), host64(y), host64(v), 1e-6)
    _, Ro, So = oracle.decode_step(q, k, v, W, feat)
    check(("first token R", dt, feat), host64(R), Ro, TOL_STATE)
    check(("first token S", dt, feat), host64(S), So, TOL_STATE)


@pytest.mark.parametrize("dt,feat,d,M", [("bf16", "favor", 64, 256), ("f32", "favor", 32, 64),
                                         ("bf16", "elu1", 128, 128)])
def test_decode_run_equals_chunked_forward_and_oracle(dt, feat, d, M):
    # T decode steps in place == one chunked forward over the T tokens == the definition
    B, H, T = 2, 3, 40
    print("decode run", dt, feat, d, M, flush=True)
    t = inputs(B, H, T, d, M, DT[dt], feat, seed=34, dy=False)
    R0, S0 = _state(B, H, d, M, dt, feat, 35, t["W"])
    R, S = R0.clone(), S0.clone()
    ys = []
    for l in range(T):
        tok = [t[n][:, :, l, :].contiguous() for n in ("q", "k", "v")]
        y, R_, S_ = A.decode_step(*tok, t["W"], feat, R, S, inplace=True)
        assert R_ is R and S_ is S
        ys.append(y)
    Yd = torch.stack(ys, dim=2)
    Yc, Rc, Sc = A.attn_fwd(t["q"], t["k"], t["v"], t["W"], feat, num_chunks=3, R_in=R0, S_in=S0)
    torch.cuda.synchronize()
    Yo, _, Ro, So = oracle.attn_fwd(t["q"], t["k"], t["v"], t["W"], feat, R0=host64(R0), S0=host64(S0))
    tol = TOL[DT[dt]]
    check(("decode run Y", dt, feat, d, M), host64(Yd), Yo, tol)
    check(("chunked Y", dt, feat, d, M), host64(Yc), Yo, tol)
    check(("decode run R", dt, feat, d, M), host64(R), Ro, TOL_STATE)
    check(("decode run S", dt, feat, d, M), host64(S), So, TOL_STATE)
    # the chunked forward multiplies bf16 copies of the features on the matrix cores, so
    # its state carries bf16 rounding; the decode step keeps them in fp32
    assert relerr_heads(host64(R), host64(Rc)) < tol


def test_in_place_equals_out_of_place():
    B, H, d, M = 2, 4, 64, 256
    q, k, v, W = _token(B, H, d, M, "bf16", "favor", seed=36)
    R, S = _state(B, H, d, M, "bf16", "favor", 37, W)
    y1, R1, S1 = A.decode_step(q, k, v, W, "favor", R, S)
    y2, R2, S2 = A.decode_step(q, k, v, W, "favor", R.clone(), S.clone(), inplace=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(R1, R2) and torch.equal(S1, S2)


def test_wide_query_range():
    # large query projections: the per-token query offset keeps g(q) finite
    B, H, d, M = 1, 4, 64, 256
    q, k, v, W = _token(B, H, d, M, "f32", "favor", seed=38)
    q = (q * 12.0).contiguous()
    R, S = _state(B, H, d, M, "f32", "favor", 39, W)
    y, R2, S2 = A.decode_step(q, k, v, W, "favor", R, S)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    yo, _, _ = oracle.decode_step(q, k, v, W, "favor", host64(R), host64(S))
    check("wide query range y", host64(y), yo, 1e-4)


def test_many_heads():
    # more heads than one grid dimension of the chunked path allows (65535)
    B, H, d, M = 300, 256, 16, 16
    q, k, v, W = _token(B, H, d, M, "bf16", "favor", seed=40)
    R = torch.rand((B, H, d, M), device="cuda") - 0.5
    S = torch.rand((B, H, M), device="cuda") + 0.5
    y, R2, S2 = A.decode_step(q, k, v, W, "favor", R, S)
    torch.cuda.synchronize()
    idx = np.random.default_rng(0).choice(B * H, 64, replace=False)
    sel = lambda x: host64(x).reshape((B * H,) + tuple(x.shape[2:]))[idx][:, None]  # noqa: E731
    yo, Ro, So = oracle.decode_step(sel(q), sel(k), sel(v), W, "favor", sel(R), sel(S))
    check("many heads y", sel(y), yo, TOL[torch.bfloat16])
    check("many heads R", sel(R2), Ro, TOL_STATE)
    check("many heads S", sel(S2), So, TOL_STATE)


@pytest.mark.parametrize("dt,feat,d,M", [("bf16", "favor", 64, 256), ("f32", "favor", 16, 32),
                                         ("f32", "elu1", 128, 128), ("bf16", "favor", 128, 64)])
def test_fp64_state_matches_oracle(dt, feat, d, M):
    # fp64 states: the update R + v g(k)^T, S + g(k) is taken in fp64, so the
    # state is the oracle's up to the fp32 rounding of the features themselves
    B, H = 2, 3
    print("decode f64", dt, feat, d, M, flush=True)
    q, k, v, W = _token(B, H, d, M, dt, feat, seed=41)
    R, S = (t.double() for t in _state(B, H, d, M, dt, feat, 42, W))
    y, R2, S2 = A.decode_step(q, k, v, W, feat, R, S)
    torch.cuda.synchronize()
    assert R2.dtype == torch.float64 and S2.dtype == torch.float64
    sc = np.exp(gpu_koff(W))
    yo, Ro, So = oracle.decode_step(q, k, v, W, feat, host64(R) * sc, host64(S) * sc)
    check(("fp64 decode y", dt, feat, d, M), host64(y), yo, TOL[DT[dt]])
    check(("fp64 decode R", dt, feat, d, M), host64(R2) * sc, Ro, TOL_STATE)
    check(("fp64 decode S", dt, feat, d, M), host64(S2) * sc, So, TOL_STATE)
    # the first token, with the state dtype asked for
    y1, R1, S1 = A.decode_step(q, k, v, W, feat, state_dtype=torch.float64)
    torch.cuda.synchronize()
    assert R1.dtype == torch.float64
    _, Ro1, So1 = oracle.decode_step(q, k, v, W, feat)
    check(("fp64 first token R", dt, feat, d, M), host64(R1) * sc, Ro1, TOL_STATE)
    check(("fp64 first token S", dt, feat, d, M), host64(S1) * sc, So1, TOL_STATE)


def test_fp64_state_keeps_small_increments():
    # after a very long prefix the state is large and one token's increment is
    # below fp32's resolution of it; an fp64 state still records the increment
    B, H, d, M = 2, 2, 64, 128
    q, k, v, W = _token(B, H, d, M, "f32", "favor", seed=43)
    rng = np.random.default_rng(44)
    R = torch.from_numpy(rng.standard_normal((B, H, d, M)) * 1e7 + 3e8).cuda()
    S = torch.from_numpy(np.abs(rng.standard_normal((B, H, M))) * 1e7 + 3e8).cuda()
    _, R2, S2 = A.decode_step(q, k, v, W, "favor", R, S)
    _, R2f, S2f = A.decode_step(q, k, v, W, "favor", R.float(), S.float())
    torch.cuda.synchronize()
    _, Ro, So = oracle.decode_step(q, k, v, W, "favor", host64(R), host64(S))
    inc_o = Ro - host64(R)
    check("fp64 increment R", host64(R2) - host64(R), inc_o, 1e-5)
    check("fp64 increment S", host64(S2) - host64(S), So - host64(S), 1e-5)
    # the fp32 state loses it (its spacing at 3e8 is 32, the increments are O(1))
    assert relerr_heads(host64(R2f) - host64(R.float()), inc_o) > 1e-1


def test_fp64_decode_run_equals_fp64_chunked_forward():
    B, H, T, d, M = 2, 3, 40, 64, 256
    t = inputs(B, H, T, d, M, torch.bfloat16, "favor", seed=45, dy=False)
    R0, S0 = (x.double() for x in _state(B, H, d, M, "bf16", "favor", 46, t["W"]))
    R, S = R0.clone(), S0.clone()
    ys = []
    for l in range(T):
        tok = [t[n][:, :, l, :].contiguous() for n in ("q", "k", "v")]
        y, _, _ = A.decode_step(*tok, t["W"], "favor", R, S, inplace=True)
        ys.append(y)
    Yd = torch.stack(ys, dim=2)
    Yc, Rc, Sc = A.attn_fwd(t["q"], t["k"], t["v"], t["W"], "favor", num_chunks=4, R_in=R0, S_in=S0)
    torch.cuda.synchronize()
    assert Rc.dtype == torch.float64
    Yo, _, Ro, So = oracle.attn_fwd(t["q"], t["k"], t["v"], t["W"], "favor", R0=host64(R0), S0=host64(S0))
    tol = TOL[torch.bfloat16]
    check("fp64 decode run Y", host64(Yd), Yo, tol)
    check("fp64 chunked Y", host64(Yc), Yo, tol)
    check("fp64 decode run R", host64(R), Ro, TOL_STATE)
    check("fp64 decode run S", host64(S), So, TOL_STATE)
    assert relerr_heads(host64(R), host64(Rc)) < tol and relerr_heads(host64(S), host64(Sc)) < tol
