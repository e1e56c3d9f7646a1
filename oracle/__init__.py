"""Python front end of the fp64 CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP product
path (``causal_linear_attention_amd``) never imports it, and the two share no
code: the only thing both sides see is the seeded input generator
(``causal_linear_attention_amd.synth``), which holds none of the method's
arithmetic.

All functions take NumPy (or anything ``np.asarray`` accepts) arrays shaped
``[B, H, L, d]`` for Q/K/V/dY, ``[M, d]`` for W, ``[B, H, d, M]`` for states R
and ``[B, H, M]`` for S, convert them to float64 and run the C code one
(batch, head) at a time, spread over a thread pool (the C calls release the
GIL).  The arithmetic of every head is sequential and unchanged by threading.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

FEAT_FAVOR = 0
FEAT_ELU1 = 1
_FEAT = {"favor": FEAT_FAVOR, "elu1": FEAT_ELU1}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle.c with gcc (IEEE fp64, no fast-math)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


_lib = None


def load(path: str | None = None):
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        _lib = _bind(ctypes.CDLL(build()))
    return _lib


_D = ctypes.POINTER(ctypes.c_double)
_Lp = ctypes.POINTER(ctypes.c_long)


def _bind(lib):
    i, l = ctypes.c_int, ctypes.c_long
    sig = {
        "oracle_featmap": [i, l, i, i, _D, _D, _D],
        "oracle_featmap_vjp": [i, l, i, i, _D, _D, _D, _D],
        "oracle_fwd_quadratic": [i, l, i, i, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D],
        "oracle_featmap_wgrad": [l, i, i, _D, _D, _D, _D],
        "oracle_bwd_quadratic": [i, l, i, i, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D],
        "oracle_fwd_prefix": [i, l, i, i, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D],
        "oracle_bwd_prefix": [i, l, i, i, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D],
        "oracle_fwd_rows": [i, l, i, i, _D, _D, _D, _D, _D, _D, l, _Lp, _D, _D],
        "oracle_softmax_fwd": [l, i, _D, _D, _D, _D],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = None
    return lib


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(_D)


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor -> numpy (float64), via CPU
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _kind(feat):
    return _FEAT[feat] if isinstance(feat, str) else int(feat)


def _threads(threads):
    return threads or min(32, os.cpu_count() or 1)


def featmap(X, W, feat="favor", M=None):
    """g(X) row by row; X [..., d] -> [..., M]."""
    lib = load()
    X = _f64(X)
    d = X.shape[-1]
    kind = _kind(feat)
    W = _f64(W) if kind == FEAT_FAVOR else np.zeros((1, d))
    M = W.shape[0] if kind == FEAT_FAVOR else d
    rows = int(np.prod(X.shape[:-1]))
    out = np.empty(X.shape[:-1] + (M,), dtype=np.float64)
    lib.oracle_featmap(kind, rows, d, M, _p(X), _p(W), _p(out))
    return out


def featmap_vjp(X, W, dPhi, feat="favor"):
    lib = load()
    X, dPhi = _f64(X), _f64(dPhi)
    d = X.shape[-1]
    kind = _kind(feat)
    W = _f64(W) if kind == FEAT_FAVOR else np.zeros((1, d))
    M = dPhi.shape[-1]
    rows = int(np.prod(X.shape[:-1]))
    out = np.empty_like(X)
    lib.oracle_featmap_vjp(kind, rows, d, M, _p(X), _p(W), _p(dPhi), _p(out))
    return out


def featmap_wgrad(X, W, dPhi):
    """FAVOR+ projection gradient of feature rows: sum over rows r of
    J_W(g(X_r))^T dPhi_r, i.e. dW[m] = sum_r dPhi[r, m] g(X_r)_m X_r  ([M, d])."""
    lib = load()
    X, W, dPhi = _f64(X), _f64(W), _f64(dPhi)
    d = X.shape[-1]
    M = W.shape[0]
    rows = int(np.prod(X.shape[:-1]))
    out = np.zeros((M, d))
    lib.oracle_featmap_wgrad(rows, d, M, _p(X), _p(W), _p(dPhi), _p(out))
    return out


def _heads(Q):
    B, H = Q.shape[0], Q.shape[1]
    return [(b, h) for b in range(B) for h in range(H)]


def attn_fwd(Q, K, V, W=None, feat="favor", R0=None, S0=None, form="quadratic", threads=None):
    """Causal linear attention forward.  Returns (Y, den, Rout, Sout).

    form="quadratic": the masked O(L^2) definition; form="prefix": the
    iterative prefix-sum recurrence."""
    lib = load()
    Q, K, V, R0, S0 = map(_f64, (Q, K, V, R0, S0))
    kind = _kind(feat)
    B, H, L, d = Q.shape
    W = _f64(W) if kind == FEAT_FAVOR else np.zeros((1, d))
    M = W.shape[0] if kind == FEAT_FAVOR else d
    Y = np.empty((B, H, L, d))
    den = np.empty((B, H, L))
    R = np.empty((B, H, d, M))
    S = np.empty((B, H, M))
    fn = lib.oracle_fwd_quadratic if form == "quadratic" else lib.oracle_fwd_prefix

    def run(bh):
        b, h = bh
        fn(kind, L, d, M, _p(Q[b, h]), _p(K[b, h]), _p(V[b, h]), _p(W),
           _p(None if R0 is None else R0[b, h]), _p(None if S0 is None else S0[b, h]),
           _p(Y[b, h]), _p(den[b, h]), _p(R[b, h]), _p(S[b, h]))

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(run, _heads(Q)))
    return Y, den, R, S


def attn_bwd(Q, K, V, W, dY, feat="favor", R0=None, S0=None, dRout=None, dSout=None,
             form="quadratic", threads=None, want_dw=False):
    """Gradients of <dY,Y> + <dRout,Rout> + <dSout,Sout>.

    Returns (dQ, dK, dV, dR0, dS0), and with want_dw (FAVOR+) also dW [M, d],
    the gradient w.r.t. the projection W shared by every batch row and head
    (the heads' contributions summed in (b, h) order)."""
    lib = load()
    Q, K, V, dY, R0, S0, dRout, dSout = map(_f64, (Q, K, V, dY, R0, S0, dRout, dSout))
    kind = _kind(feat)
    B, H, L, d = Q.shape
    W = _f64(W) if kind == FEAT_FAVOR else np.zeros((1, d))
    M = W.shape[0] if kind == FEAT_FAVOR else d
    dQ, dK, dV = (np.empty((B, H, L, d)) for _ in range(3))
    dR0 = np.empty((B, H, d, M))
    dS0 = np.empty((B, H, M))
    if want_dw and kind != FEAT_FAVOR:
        raise ValueError("dW exists only for the FAVOR+ feature map")
    dWh = np.zeros((B, H, M, d)) if want_dw else None
    fn = lib.oracle_bwd_quadratic if form == "quadratic" else lib.oracle_bwd_prefix

    def sel(a, b, h):
        return None if a is None else a[b, h]

    def run(bh):
        b, h = bh
        fn(kind, L, d, M, _p(Q[b, h]), _p(K[b, h]), _p(V[b, h]), _p(W),
           _p(sel(R0, b, h)), _p(sel(S0, b, h)), _p(dY[b, h]),
           _p(sel(dRout, b, h)), _p(sel(dSout, b, h)),
           _p(dQ[b, h]), _p(dK[b, h]), _p(dV[b, h]), _p(dR0[b, h]), _p(dS0[b, h]),
           _p(sel(dWh, b, h)))

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(run, _heads(Q)))
    if not want_dw:
        return dQ, dK, dV, dR0, dS0
    dW = np.zeros((M, d))
    for b, h in _heads(Q):
        dW += dWh[b, h]
    return dQ, dK, dV, dR0, dS0, dW


def attn_fwd_rows(Q, K, V, W, rows, feat="favor", R0=None, S0=None):
    """Y_l and den_l by the definition for the listed rows of ONE head.

    Q, K, V: [L, d]; rows: 1-D integer array.  Returns (Yrows [n, d], den [n])."""
    lib = load()
    Q, K, V, R0, S0 = map(_f64, (Q, K, V, R0, S0))
    kind = _kind(feat)
    L, d = Q.shape
    W = _f64(W) if kind == FEAT_FAVOR else np.zeros((1, d))
    M = W.shape[0] if kind == FEAT_FAVOR else d
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    Yr = np.empty((rows.size, d))
    dr = np.empty(rows.size)
    lib.oracle_fwd_rows(kind, L, d, M, _p(Q), _p(K), _p(V), _p(W), _p(R0), _p(S0),
                        rows.size, rows.ctypes.data_as(_Lp), _p(Yr), _p(dr))
    return Yr, dr


def decode_step(q, k, v, W=None, feat="favor", R0=None, S0=None):
    """One position of the iterative prefix-sum evaluation (eq. (3)-(4) of
    Subsection 2.1, walked one token at a time): q, k, v [B, H, d], state
    R0 [B, H, d, M], S0 [B, H, M] (None = zero).  Returns (y [B, H, d], R, S),
    the output for the new token and the state after it.  It is the prefix
    form run over a sequence of length one from the given state."""
    q, k, v = (_f64(t)[:, :, None, :] for t in (q, k, v))
    Y, _, R, S = attn_fwd(q, k, v, W, feat, R0, S0, form="prefix")
    return Y[:, :, 0, :], R, S


def softmax_fwd(Q, K, V, threads=None):
    """Causal exponential attention (no temperature); [B, H, L, d] -> Y."""
    lib = load()
    Q, K, V = map(_f64, (Q, K, V))
    B, H, L, d = Q.shape
    Y = np.empty((B, H, L, d))

    def run(bh):
        b, h = bh
        lib.oracle_softmax_fwd(L, d, _p(Q[b, h]), _p(K[b, h]), _p(V[b, h]), _p(Y[b, h]))

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(run, _heads(Q)))
    return Y
