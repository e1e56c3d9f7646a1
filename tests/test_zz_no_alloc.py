"""The allocation-free forward (slim_attn_fwd_noalloc) against slim_attn_fwd, through
the C ABI, on two calls in a row, the second with a smaller input.

slim_attn_fwd_noalloc works in a fixed 64 MiB device array instead of a caller's
workspace.  The first call (the 16K-token, 64-head workload's shape, one slice per
workgroup: its automatic window, all 32 slices, needs 140 MB of slots) has to shrink
its window to fit, so it runs in several windows: its outputs are bitwise those of
slim_attn_fwd given the same window, and within the bf16 bound (2e-2, gpu_util.check)
of slim_attn_fwd with the automatic window and of the fp64 oracle on sampled heads.  The second call (smaller,
fp32) fits whole: bitwise equal to slim_attn_fwd.  Both calls share the array, so the
second also shows that nothing left in it by the first leaks into its result."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from causal_linear_attention_amd import _lib
from causal_linear_attention_amd import attention as A
from gpu_util import TOL, check, host64, inputs

pytestmark = pytest.mark.gpu


def _noalloc_window(q, M, feat, C, G=0):
    """The window slim_attn_fwd_noalloc takes: the largest whose forward workspace fits."""
    P = int(_lib.lib().slim_window_chunks(ctypes.byref(A.make_desc(q, M, feat, C, group_slices=G))))
    while P > 1 and A.workspace_bytes(A.make_desc(q, M, feat, C, P, group_slices=G), _lib.SLIM_PASS_FWD) > \
            _lib.SLIM_NOALLOC_SCRATCH_BYTES:
        P -= 1
    return P


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


def test_noalloc_forward_two_calls():
    # call 1: B=4, H=16, L=16384, d=64, M=256, bf16, 32 slices of 512, one per workgroup
    B, H, L, d, M, C, G = 4, 16, 16384, 64, 256, 32, 1
    print("no-alloc forward, call 1", (B, H, L, d, M, C), flush=True)
    x = inputs(B, H, L, d, M, torch.bfloat16, "favor", seed=81, dy=False)
    ko = torch.full((1,), -1.0, device="cuda")
    got = A.attn_fwd_noalloc(x["q"], x["k"], x["v"], x["W"], "favor", C, want_row_stats=True, koff_out=ko,
                             group_slices=G)
    P = _noalloc_window(x["q"], M, "favor", C, G)
    assert P < C  # the automatic window does not fit the array: several windows
    same_window = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", C, window_chunks=P, want_row_stats=True,
                             group_slices=G)
    auto = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", C, want_row_stats=True, group_slices=G)
    torch.cuda.synchronize()
    print("window", P, "of", C, "slices", flush=True)
    assert float(ko) == 0.0
    assert _same(got, same_window)
    tol = TOL[torch.bfloat16]
    for nm, g, a in zip(("Y", "R", "S", "row stats"), got, auto):
        check(("no-alloc vs slim_attn_fwd", nm), host64(g), host64(a), tol)
    # and the oracle on sampled heads (its prefix form)
    sel = [(0, 0), (B - 1, H - 1)]
    h = {n: np.stack([host64(x[n][b, hh]) for b, hh in sel])[None] for n in ("q", "k", "v")}
    Yo, _, Ro, So = oracle.attn_fwd(h["q"], h["k"], h["v"], host64(x["W"]), "favor", form="prefix")
    for nm, g, ref in (("Y", got[0], Yo), ("R", got[1], Ro), ("S", got[2], So)):
        gs = np.stack([host64(g[b, hh]) for b, hh in sel])[None]
        check(("no-alloc vs oracle", nm), gs, ref, tol)
    del x, got, same_window, auto

    # call 2, smaller: B=1, H=2, L=300, d=64, M=64, fp32, 7 slices; fits whole
    B, H, L, d, M, C = 1, 2, 300, 64, 64, 7
    print("no-alloc forward, call 2", (B, H, L, d, M, C), flush=True)
    x = inputs(B, H, L, d, M, torch.float32, "favor", seed=82, dy=False)
    rng = np.random.default_rng(83)
    R0 = torch.from_numpy(rng.standard_normal((B, H, d, M)).astype(np.float32) * 0.1).cuda()
    S0 = torch.from_numpy(np.abs(rng.standard_normal((B, H, M))).astype(np.float32) + 0.5).cuda()
    got = A.attn_fwd_noalloc(x["q"], x["k"], x["v"], x["W"], "favor", C, R_in=R0, S_in=S0, want_row_stats=True)
    ref = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", C, R_in=R0, S_in=S0, want_row_stats=True)
    torch.cuda.synchronize()
    assert _same(got, ref)
    Yo, _, Ro, So = oracle.attn_fwd(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(x["W"]), "favor",
                                    R0=host64(R0), S0=host64(S0))
    for nm, g, r in (("Y", got[0], Yo), ("R", got[1], Ro), ("S", got[2], So)):
        check(("no-alloc call 2 vs oracle", nm), host64(g), r, TOL[torch.float32])
