"""Non-finite inputs propagate, and only along the causal dependencies (page "Sub-Linear
Memory: How to Make Performers SLiM", Subsection 2.1: Y_l depends only on indices up to
l).  The library masks nothing: a NaN or Inf in Q_j, K_j or V_j makes every output that
depends on it non-finite.  Outputs that do not depend on it are bitwise those of the
clean run, up to the granularity of a tile: inside the tile of TT rows that holds row j,
the masked (upper) triangle of a tile product multiplies the bad value by zero, which
gives NaN for the other rows of that tile too.

Dependencies (one window: the entry states are rebuilt forward, the gradient state is a
suffix sum of direct sums):
  * Q_j: Y_j; dQ_j; dK_s, dV_s for s <= j (through P[j][s], A[j][s] and the gradient
    state).  Every other row of Y and dQ is exact, and dK, dV after j's tile.
  * K_j: Y_l for l >= j (through the state), hence the denominators and dNum of those
    rows, every dK and dV (through the gradient state of every earlier slice), and dQ_l
    for l >= j.  Y and dQ before j's tile are exact.
  * V_j: as K_j, except that the denominators do not involve V, and neither does dV
    (Y is linear in V): dV is exact everywhere.
With several windows, the backward recovers each window's start state by subtraction
(update (19)), so a bad K_j or V_j reaches every entry state of the sequence; the Q_j
case is the same as with one window."""
import pytest
import torch

from causal_linear_attention_amd import attention as A
from gpu_util import DT, inputs

pytestmark = pytest.mark.gpu

B, H, L, d, M, C = 1, 2, 2048, 64, 128, 4
J = 1000  # the bad row: inside slice 1 (rows 512..1023) and inside the tile 992..1023


def _rows_finite(t):
    """[B, H, L] bool: every element of the row is finite."""
    return torch.isfinite(t).all(dim=-1)


def _run(x, window):
    Y, R, S, rs = A.attn_fwd(x["q"], x["k"], x["v"], x["W"], "favor", C, window_chunks=window, want_row_stats=True)
    g = A.attn_bwd(x["q"], x["k"], x["v"], x["W"], x["dy"], "favor", C, window_chunks=window, Y=Y, row_stats=rs)
    torch.cuda.synchronize()
    return {"Y": Y, "dQ": g[0], "dK": g[1], "dV": g[2]}


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("bad", [float("nan"), float("inf")], ids=["nan", "inf"])
@pytest.mark.parametrize("where", ["q", "k", "v"])
@pytest.mark.parametrize("window", [0, 1], ids=["one_window", "four_windows"])
def test_nonfinite_input_propagates_along_dependencies(dt, bad, where, window):
    x = inputs(B, H, L, d, M, DT[dt], "favor", seed=71)
    tt = int(A._lib.lib().slim_tile_rows(A.make_desc(x["q"], M, "favor", C)))
    assert tt == 32
    t0, t1 = J - J % tt, J - J % tt + tt  # the bad row's tile
    clean = _run(x, window)
    y = dict(x)
    t = x[where].clone()
    t[:, :, J, 5] = bad
    y[where] = t
    dirty = _run(y, window)
    print("non-finite", dt, bad, where, "window", window, flush=True)
    rows = torch.arange(L, device="cuda")
    every, none = rows >= 0, rows < 0
    for name in ("Y", "dQ", "dK", "dV"):
        a, b = clean[name], dirty[name]
        fin = _rows_finite(b)
        if where == "q":
            exact = rows != J if name in ("Y", "dQ") else rows >= t1
            affected = rows == J if name in ("Y", "dQ") else rows <= J
        elif name == "Y":
            exact, affected = rows < t0, rows >= J
        elif name == "dQ":  # several windows: the start states come from subtraction
            exact, affected = (rows < t0) if window == 0 else none, rows >= J
        elif name == "dV" and where == "v":
            exact, affected = every, none
        else:
            exact, affected = none, every
        # the bad value is not masked: every row that depends on it is non-finite
        assert not bool(fin[:, :, affected].any()), (name, "a dependent row stayed finite")
        # and every row that does not (outside its tile) is exactly the clean result
        assert torch.equal(a[:, :, exact], b[:, :, exact]), (name, "an independent row changed")
