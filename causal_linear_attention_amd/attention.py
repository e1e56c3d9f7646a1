"""PyTorch front end of libslim: device memory, streams and autograd wiring.

Every step of the computation runs in the HIP kernels behind the C ABI; this
module only checks tensors, allocates outputs/workspace with PyTorch's caching
allocator (so ``torch.cuda.max_memory_allocated`` sees all of it) and passes
pointers plus the current stream.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

_DT = {torch.float32: _lib.SLIM_F32, torch.bfloat16: _lib.SLIM_BF16}
_SDT = {torch.float32: _lib.SLIM_F32, torch.float64: _lib.SLIM_F64}  # state element types
_FEAT = {"favor": _lib.SLIM_FEAT_FAVOR, "elu1": _lib.SLIM_FEAT_ELU1}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_io(name, t, dtype, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def make_desc(q, M, feat, num_chunks, window_chunks=0, state_dtype=torch.float32, group_slices=0):
    B, H, L, d = q.shape
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if state_dtype not in _SDT:
        raise ValueError(f"unsupported state dtype {state_dtype}")
    return _lib.desc(B, H, L, d, M, num_chunks, window_chunks, _DT[q.dtype], _FEAT[feat], _SDT[state_dtype],
                     group_slices)


def _feat_M(W, feat, d):
    if feat == "favor":
        if W is None:
            raise ValueError("FAVOR+ needs W")
        return W.shape[0]
    if W is not None:
        raise ValueError("elu1 takes no W")
    return d


def workspace_bytes(desc, pass_, states=False):
    """Workspace bytes of a pass; states: with a states buffer given to the call."""
    fn = _lib.lib().slim_workspace_bytes_states if states else _lib.lib().slim_workspace_bytes
    n = fn(ctypes.byref(desc), pass_)
    if n == 0 and pass_ != _lib.SLIM_PASS_FEATMAP:
        _lib.check(_lib.lib().slim_validate(ctypes.byref(desc), pass_), "slim_workspace_bytes")
    return n


def state_shape(dsc):
    """Shape of the per-group states attn_fwd(want_states=True) returns for a
    descriptor: one entry per group of slices (slim_group_slices) and the final state."""
    c = -(-dsc.L // dsc.num_chunks)
    G = _lib.lib().slim_group_slices(ctypes.byref(dsc))
    return (dsc.B, dsc.H, -(-dsc.L // min(c * G, dsc.L)) + 1, dsc.d + 1, dsc.M)


def featmap(x, W=None, feat="favor", row_offset=False):
    """g(x) in fp32: x [B, H, L, d] -> [B, H, L, M] (and the per-row offsets)."""
    B, H, L, d = x.shape
    M = _feat_M(W, feat, d)
    _check_io("x", x, x.dtype)
    if W is not None:
        _check_io("W", W, x.dtype, (M, d))
    dsc = make_desc(x, M, feat, 1)
    phi = torch.empty((B, H, L, M), dtype=torch.float32, device=x.device)
    off = torch.empty((B, H, L), dtype=torch.float32, device=x.device) if row_offset else None
    _lib.check(_lib.lib().slim_featmap(ctypes.byref(dsc), _ptr(x), _ptr(W), _ptr(phi), _ptr(off), _stream()),
               "slim_featmap")
    return (phi, off) if row_offset else phi


def attn_fwd(q, k, v, W=None, feat="favor", num_chunks=1, R_in=None, S_in=None, window_chunks=0,
             state_dtype=None, want_row_stats=False, koff_out=None, want_states=False, group_slices=0):
    """Forward.  Returns (Y, R_out [B,H,d,M], S_out [B,H,M]).  States are fp32, or
    fp64 when R_in is fp64 or state_dtype=torch.float64; like R_in, S_in they hold
    the state times exp(-koff), the key-side offset of W (0 unless some row of W has
    |w_m|^2 > 120).  want_row_stats: a fourth value, the per-row statistics
    [B,H,L,2] fp32 that let attn_bwd skip recomputing the denominators (pass it
    with Y).  want_states: a fifth value (the fourth None unless want_row_stats),
    the state entering every group of slices [B,H,groups+1,d+1,M] fp32 (rows < d:
    R, row d: S, times exp(-koff)) for attn_bwd to read instead of rebuilding them,
    or None where the slices span several windows.  koff_out: a one-element fp32
    GPU tensor that receives koff.  group_slices: consecutive slices one workgroup
    walks (0 = automatic, 1 = one slice each); pass the same to attn_bwd."""
    B, H, L, d = q.shape
    M = _feat_M(W, feat, d)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_io(n, t, q.dtype, q.shape)
    if W is not None:
        _check_io("W", W, q.dtype, (M, d))
    sd = R_in.dtype if R_in is not None else (state_dtype or torch.float32)
    if R_in is not None:
        _check_io("R_in", R_in, sd, (B, H, d, M))
        _check_io("S_in", S_in, sd, (B, H, M))
    dsc = make_desc(q, M, feat, num_chunks, window_chunks, sd, group_slices)
    st = None
    if want_states and _lib.lib().slim_state_bytes(ctypes.byref(dsc)) > 0:
        st = torch.empty(state_shape(dsc), dtype=torch.float32, device=q.device)
        assert st.numel() * 4 == _lib.lib().slim_state_bytes(ctypes.byref(dsc))
    ws = torch.empty(max(1, workspace_bytes(dsc, _lib.SLIM_PASS_FWD, st is not None)), dtype=torch.uint8,
                     device=q.device)
    Y = torch.empty_like(q)
    R = torch.empty((B, H, d, M), dtype=sd, device=q.device)
    S = torch.empty((B, H, M), dtype=sd, device=q.device)
    rs = torch.empty((B, H, L, 2), dtype=torch.float32, device=q.device) if want_row_stats else None
    if koff_out is not None:
        _check_io("koff_out", koff_out, torch.float32, (1,))
    _lib.check(_lib.lib().slim_attn_fwd(ctypes.byref(dsc), _ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(R_in),
                                        _ptr(S_in), _ptr(Y), _ptr(R), _ptr(S), _ptr(koff_out), _ptr(rs), _ptr(st),
                                        _ptr(ws), ws.numel(), _stream()),
               "slim_attn_fwd")
    if want_states:
        return Y, R, S, rs, st
    if want_row_stats:
        return Y, R, S, rs
    return Y, R, S


def attn_fwd_noalloc(q, k, v, W=None, feat="favor", num_chunks=1, R_in=None, S_in=None, window_chunks=0,
                     state_dtype=None, want_row_stats=False, koff_out=None, out=None, group_slices=0):
    """attn_fwd through slim_attn_fwd_noalloc: the library allocates no workspace (it
    works in its own fixed device array).  out: optional (Y, R_out, S_out[, row_stats])
    tensors to write into, so that a caller can avoid every allocation; else they are
    allocated here.  Same results as attn_fwd."""
    B, H, L, d = q.shape
    M = _feat_M(W, feat, d)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_io(n, t, q.dtype, q.shape)
    if W is not None:
        _check_io("W", W, q.dtype, (M, d))
    sd = R_in.dtype if R_in is not None else (state_dtype or torch.float32)
    if R_in is not None:
        _check_io("R_in", R_in, sd, (B, H, d, M))
        _check_io("S_in", S_in, sd, (B, H, M))
    dsc = make_desc(q, M, feat, num_chunks, window_chunks, sd, group_slices)
    if out is None:
        Y = torch.empty_like(q)
        R = torch.empty((B, H, d, M), dtype=sd, device=q.device)
        S = torch.empty((B, H, M), dtype=sd, device=q.device)
        rs = torch.empty((B, H, L, 2), dtype=torch.float32, device=q.device) if want_row_stats else None
    else:
        Y, R, S = out[:3]
        rs = out[3] if len(out) > 3 else None
        _check_io("Y", Y, q.dtype, q.shape)
        _check_io("R_out", R, sd, (B, H, d, M))
        _check_io("S_out", S, sd, (B, H, M))
        if rs is not None:
            _check_io("row_stats", rs, torch.float32, (B, H, L, 2))
    if koff_out is not None:
        _check_io("koff_out", koff_out, torch.float32, (1,))
    _lib.check(_lib.lib().slim_attn_fwd_noalloc(ctypes.byref(dsc), _ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(R_in),
                                                _ptr(S_in), _ptr(Y), _ptr(R), _ptr(S), _ptr(koff_out), _ptr(rs),
                                                _stream()),
               "slim_attn_fwd_noalloc")
    if rs is not None:
        return Y, R, S, rs
    return Y, R, S


def attn_bwd(q, k, v, W, dY, feat="favor", num_chunks=1, R_in=None, S_in=None, dR_out=None, dS_out=None,
             want_state_grad=False, window_chunks=0, state_dtype=None, want_dw=False, Y=None, row_stats=None,
             states=None, group_slices=0):
    """Backward of attn_fwd(q, k, v, W, feat, num_chunks, R_in, S_in) for the
    loss <dY, Y> + <dR_out, R_out> + <dS_out, S_out>.  Returns (dQ, dK, dV,
    dR_in, dS_in); the last two are None unless want_state_grad.  With want_dw
    (FAVOR+) a sixth value follows: dW [M, d] fp32, the gradient w.r.t. the
    projection W.  The state tensors share one dtype (fp32, or fp64), taken
    from those given.  Y, row_stats: the output and row statistics of attn_fwd on
    the same inputs (want_row_stats=True); given, the backward reuses the
    forward's denominators instead of recomputing them.  states: what
    attn_fwd(want_states=True) returned for the same inputs and slices; the
    backward then reads every slice's entry state instead of rebuilding it
    (same results)."""
    B, H, L, d = q.shape
    M = _feat_M(W, feat, d)
    for n, t in (("q", q), ("k", k), ("v", v), ("dY", dY)):
        _check_io(n, t, q.dtype, q.shape)
    given = [t for t in (R_in, dR_out) if t is not None]
    sd = given[0].dtype if given else (state_dtype or torch.float32)
    if R_in is not None:
        _check_io("R_in", R_in, sd, (B, H, d, M))
        _check_io("S_in", S_in, sd, (B, H, M))
    if dR_out is not None:
        _check_io("dR_out", dR_out, sd, (B, H, d, M))
        _check_io("dS_out", dS_out, sd, (B, H, M))
    if want_dw and feat != "favor":
        raise ValueError("dW exists only for the FAVOR+ feature map")
    if (Y is None) != (row_stats is None):
        raise ValueError("give both Y and row_stats, or neither")
    if Y is not None:
        _check_io("Y", Y, q.dtype, q.shape)
        _check_io("row_stats", row_stats, torch.float32, (B, H, L, 2))
    dsc = make_desc(q, M, feat, num_chunks, window_chunks, sd, group_slices)
    if states is not None:
        _check_io("states", states, torch.float32, state_shape(dsc))
    ps = _lib.SLIM_PASS_BWD_DW if want_dw else _lib.SLIM_PASS_BWD
    ws = torch.empty(max(1, workspace_bytes(dsc, ps, states is not None)), dtype=torch.uint8, device=q.device)
    dQ, dK, dV = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dW = torch.empty((M, d), dtype=torch.float32, device=q.device) if want_dw else None
    dR = dS = None
    if want_state_grad:
        dR = torch.empty((B, H, d, M), dtype=sd, device=q.device)
        dS = torch.empty((B, H, M), dtype=sd, device=q.device)
    _lib.check(_lib.lib().slim_attn_bwd(ctypes.byref(dsc), _ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(dY),
                                        _ptr(Y), _ptr(row_stats), _ptr(states), _ptr(R_in), _ptr(S_in), _ptr(dR_out),
                                        _ptr(dS_out), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dR), _ptr(dS), _ptr(dW),
                                        _ptr(ws), ws.numel(), _stream()),
               "slim_attn_bwd")
    if want_dw:
        return dQ, dK, dV, dR, dS, dW
    return dQ, dK, dV, dR, dS


def decode_step(q, k, v, W=None, feat="favor", R=None, S=None, inplace=False, state_dtype=None):
    """One recurrent decode step for one new token per head.

    q, k, v: [B, H, d] (fp32 or bf16); R [B, H, d, M], S [B, H, M] (fp32, or fp64):
    the state before the token (None = zero, the first token).  Returns (y, R', S')
    with y [B, H, d] and R' = R + v g(k)^T, S' = S + g(k), in the state's dtype
    (R's, else state_dtype, else fp32).  inplace=True writes R', S' into R, S (which
    must be given) and returns them."""
    if q.dim() != 3:
        raise ValueError("decode_step takes q, k, v of shape [B, H, d]")
    B, H, d = q.shape
    M = _feat_M(W, feat, d)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_io(n, t, q.dtype, q.shape)
    if W is not None:
        _check_io("W", W, q.dtype, (M, d))
    if (R is None) != (S is None):
        raise ValueError("give both R and S, or neither")
    sd = R.dtype if R is not None else (state_dtype or torch.float32)
    if sd not in _SDT:
        raise ValueError(f"unsupported state dtype {sd}")
    if R is not None:
        _check_io("R", R, sd, (B, H, d, M))
        _check_io("S", S, sd, (B, H, M))
    elif inplace:
        raise ValueError("inplace needs R and S")
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dsc = _lib.desc(B, H, 1, d, M, 1, 0, _DT[q.dtype], _FEAT[feat], _SDT[sd])
    y = torch.empty_like(q)
    if inplace:
        Ro, So = R, S
    else:
        Ro = torch.empty((B, H, d, M), dtype=sd, device=q.device)
        So = torch.empty((B, H, M), dtype=sd, device=q.device)
    _lib.check(_lib.lib().slim_decode_step(ctypes.byref(dsc), _ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(R),
                                           _ptr(S), _ptr(y), _ptr(Ro), _ptr(So), _stream()),
               "slim_decode_step")
    return y, Ro, So


class _SlimAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, W, feat, num_chunks, window_chunks, keep_states, group_slices):
        out = attn_fwd(q, k, v, W, feat, num_chunks, window_chunks=window_chunks, want_row_stats=True,
                       want_states=keep_states, group_slices=group_slices)
        Y, rs, st = out[0], out[3], out[4] if keep_states else None
        # Kept for the backward: the inputs, the output, 8 bytes per row of
        # denominator statistics and, where one window holds every slice and
        # keep_states is set, each slice's entry state ((d+1) M fp32 per slice);
        # else the backward rebuilds the entry states.  The slices are recomputed
        # either way.
        ctx.save_for_backward(q, k, v, W if W is not None else torch.empty(0), Y, rs,
                              st if st is not None else torch.empty(0))
        ctx.feat, ctx.num_chunks, ctx.window_chunks, ctx.has_w = feat, num_chunks, window_chunks, W is not None
        ctx.has_st, ctx.group_slices = st is not None, group_slices
        return Y

    @staticmethod
    def backward(ctx, dY):
        q, k, v, W, Y, rs, st = ctx.saved_tensors
        want_dw = ctx.has_w and ctx.needs_input_grad[3]
        g = attn_bwd(q, k, v, W if ctx.has_w else None, dY.contiguous(), ctx.feat, ctx.num_chunks,
                     window_chunks=ctx.window_chunks, want_dw=want_dw, Y=Y, row_stats=rs,
                     states=st if ctx.has_st else None, group_slices=ctx.group_slices)
        dW = g[5].to(W.dtype) if want_dw else None
        return g[0], g[1], g[2], dW, None, None, None, None, None


def slim_attention(q, k, v, W=None, feat="favor", num_chunks=1, window_chunks=0, keep_states=True, group_slices=0):
    """Causal linear attention with autograd: gradients for q, k, v, and for
    the FAVOR+ projection W when it requires one (the page keeps W a fixed
    random projection; a caller may train it).  keep_states: where one window
    holds every slice, keep each slice's entry state from the forward for the
    backward ((d+1) M fp32 per group of slices and head) instead of rebuilding them.
    group_slices: consecutive slices one workgroup walks (0 = automatic)."""
    return _SlimAttention.apply(q, k, v, W, feat, num_chunks, window_chunks, keep_states, group_slices)
