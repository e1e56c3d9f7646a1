"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/slim.h declares, and its validation / workspace
planning behave as documented.  Nothing here launches a kernel."""
import ctypes
import os
import re

import pytest

from causal_linear_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "slim.h")


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(slim_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libslim.so not built")
    return _lib.lib()


def test_header_lists_the_binding_exports():
    assert header_functions() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.slim_version() >> 16 == 4
    for code in range(8):
        assert lib.slim_status_string(code)
    assert lib.slim_status_string(0) == b"ok"


def d_(**kw):
    base = dict(B=2, H=3, L=1000, d=64, M=128, num_chunks=8, window_chunks=0, dtype=_lib.SLIM_BF16,
                feat=_lib.SLIM_FEAT_FAVOR, state_dtype=_lib.SLIM_F32)
    base.update(kw)
    return _lib.desc(**base)


def validate(lib, pass_=_lib.SLIM_PASS_FWD, **kw):
    return lib.slim_validate(ctypes.byref(d_(**kw)), pass_)


def test_validate_ok(lib):
    for p in (0, 1, 2):
        assert validate(lib, p) == 0
    assert validate(lib, feat=_lib.SLIM_FEAT_ELU1, M=64) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 2), (dict(H=-1), 2), (dict(L=0), 2), (dict(num_chunks=0), 2), (dict(num_chunks=1001), 2),
    (dict(window_chunks=-1), 2), (dict(L=1 << 31), 2), (dict(dtype=7), 3), (dict(feat=9), 3),
    (dict(feat=_lib.SLIM_FEAT_ELU1), 2),            # elu+1 needs M == d
    (dict(d=48), 4), (dict(M=96), 4), (dict(M=512), 4), (dict(d=256, M=256), 4),
    (dict(B=65536, H=1), 4), (dict(B=256, H=257), 4),  # more heads than one launch's grid takes
])
def test_validate_errors(lib, kw, code):
    assert validate(lib, **kw) == code


def test_validate_null(lib):
    assert lib.slim_validate(None, 1) == 1


FWD_ARGS = ("Q", "K", "V", "W", "R_in", "S_in", "Y", "R_out", "S_out", "koff", "row_stats", "states", "ws",
            "ws_bytes", "stream")
BWD_ARGS = ("Q", "K", "V", "W", "dY", "Y", "row_stats", "states", "R_in", "S_in", "dR_out", "dS_out", "dQ", "dK",
            "dV", "dR_in", "dS_in", "dW", "ws", "ws_bytes", "stream")
P = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first


def fwd(lib, d, **kw):
    """slim_attn_fwd with the named pointers; Q, K, V, W, Y, R_out, S_out, ws default to
    a dummy address, the rest to NULL / 0."""
    base = dict(Q=P, K=P, V=P, W=P, Y=P, R_out=P, S_out=P, ws=P, ws_bytes=1 << 40)
    base.update(kw)
    return lib.slim_attn_fwd(ctypes.byref(d), *[base.get(n) for n in FWD_ARGS])


def bwd(lib, d, **kw):
    base = dict(Q=P, K=P, V=P, W=P, dY=P, dQ=P, dK=P, dV=P, ws=P, ws_bytes=1 << 40)
    base.update(kw)
    return lib.slim_attn_bwd(ctypes.byref(d), *[base.get(n) for n in BWD_ARGS])


def test_entry_points_reject_before_any_launch(lib):
    d = d_()
    # NULL inputs / workspace: rejected on the host, nothing enqueued
    nulls = {n: None for n in FWD_ARGS}
    nulls["ws_bytes"] = 0
    assert fwd(lib, d, **nulls) == 1
    assert fwd(lib, d, ws_bytes=0) == 5
    bad = ctypes.c_void_p((1 << 20) + 4)
    assert fwd(lib, d, Q=bad) == 6
    assert fwd(lib, d, row_stats=bad) == 6
    assert fwd(lib, d, koff=ctypes.c_void_p((1 << 20) + 2)) == 6
    assert bwd(lib, d_(num_chunks=0)) == 2
    # only one of the paired initial-state pointers
    assert fwd(lib, d, R_in=P) == 1
    assert bwd(lib, d, R_in=P) == 1
    # only one of the forward's output and row statistics
    assert bwd(lib, d, Y=P) == 1
    assert bwd(lib, d, row_stats=P) == 1
    assert bwd(lib, d, Y=P, row_stats=bad) == 6
    # elu+1 takes no W
    de = d_(feat=_lib.SLIM_FEAT_ELU1, M=64)
    assert fwd(lib, de) == 2
    assert lib.slim_featmap(ctypes.byref(de), P, None, P, P, None) == 2


def test_dw_pass_validation(lib):
    # the projection gradient exists for FAVOR+ only, and needs the larger workspace
    BWD, DW = _lib.SLIM_PASS_BWD, _lib.SLIM_PASS_BWD_DW
    assert validate(lib, DW) == 0
    assert validate(lib, DW, dtype=_lib.SLIM_F32, d=128, M=256) == 0
    assert validate(lib, DW, feat=_lib.SLIM_FEAT_ELU1, M=64) == 4
    assert validate(lib, 5) == 2
    assert ws(lib, DW) > ws(lib, BWD) > 0
    assert ws(lib, DW, feat=_lib.SLIM_FEAT_ELU1, M=64) == 0
    # the extra space: two [B*H][window rows][M] buffers of the io dtype plus the partial sums
    d = dict(B=2, H=3, L=4096, d=64, M=128, num_chunks=16, window_chunks=16)
    extra = ws(lib, DW, **d) - ws(lib, BWD, **d)
    assert extra >= 2 * 6 * 4096 * 128 * 2
    # bounded by the window, not by L (one slice per workgroup: the automatic grouping
    # depends on L and only shrinks the per-group buffers)
    big = [ws(lib, DW, B=1, H=8, L=n, d=64, M=64, num_chunks=n // 512, window_chunks=64, group_slices=1)
           for n in (1 << 16, 1 << 20)]
    assert big[0] == big[1]
    auto = [ws(lib, DW, B=1, H=8, L=n, d=64, M=64, num_chunks=n // 512, window_chunks=64) for n in (1 << 16, 1 << 20)]
    assert max(auto) <= big[0]


@pytest.mark.parametrize("dtype", [_lib.SLIM_F32, _lib.SLIM_BF16])
def test_automatic_window_bounds_every_pass(lib, dtype):
    # the automatic window keeps each pass's per-slice buffers within 1 GiB (with dW the
    # two rows of dg(X) . g(X) per slice row within another 1 GiB), for any L at a given
    # slice length
    GiB = 1 << 30
    for c in (512, 4096):
        sizes = {}
        for p in (_lib.SLIM_PASS_FWD, _lib.SLIM_PASS_BWD, _lib.SLIM_PASS_BWD_DW):
            sizes[p] = [ws(lib, p, dtype=dtype, B=1, H=8, L=n, d=64, M=256, num_chunks=n // c)
                        for n in (1 << 16, 1 << 20, 1 << 22, 1 << 24)]
            # per-slice buffers within the budget, plus what does not grow with L: the
            # carries, W^T and the dW partial sums (at most about 1024 fp32 [M][d] blocks)
            budget = (2 if p == _lib.SLIM_PASS_BWD_DW else 1) * GiB
            assert max(sizes[p]) <= budget + (192 << 20), (c, p, sizes[p])
            # constant once L is past what fits whole
            assert sizes[p][-1] == sizes[p][-2], (c, p, sizes[p])
    # a few long slices of many rows: the window shrinks to what fits (at least one slice)
    one = ws(lib, _lib.SLIM_PASS_BWD_DW, dtype=dtype, B=1, H=1, L=1 << 22, d=64, M=256, num_chunks=1024)
    assert 0 < one <= 2 * GiB + (192 << 20)


def test_dw_rejects_before_any_launch(lib):
    dw = ctypes.c_void_p(1 << 21)
    d = d_()
    # workspace sized for the plain backward is too small once dW is asked for
    wsb = lib.slim_workspace_bytes(ctypes.byref(d), _lib.SLIM_PASS_BWD)
    assert bwd(lib, d, dW=dw, ws_bytes=wsb) == 5
    # misaligned dW
    assert bwd(lib, d, dW=ctypes.c_void_p((1 << 21) + 4)) == 6
    # elu+1 has no projection
    de = d_(feat=_lib.SLIM_FEAT_ELU1, M=64)
    assert bwd(lib, de, W=None, dW=dw) == 4


def ws(lib, pass_, **kw):
    return lib.slim_workspace_bytes(ctypes.byref(d_(**kw)), pass_)


def test_workspace_sizes(lib):
    assert ws(lib, 0) == 0
    assert 0 < ws(lib, 1) < ws(lib, 2)
    assert ws(lib, 1, B=0) == 0
    # forward: (window + 1) slots of (d + 1) * M fp32 per head
    d = d_(L=4096, num_chunks=16, window_chunks=16)
    assert lib.slim_workspace_bytes(ctypes.byref(d), 1) >= 6 * 17 * 65 * 128 * 4


def test_workspace_does_not_grow_with_L_at_fixed_slice_and_window(lib):
    # slice length 512, window of 64 slices: once L exceeds 64 * 512 the workspace is flat
    # (one slice per workgroup); with the automatic grouping, which takes two slices per
    # workgroup once there are enough of them, it never exceeds that
    for g in (1, 0):
        sizes = [ws(lib, 2, B=1, H=8, L=n, d=64, M=64, num_chunks=n // 512, window_chunks=64, group_slices=g)
                 for n in (1 << 15, 1 << 16, 1 << 18, 1 << 20)]
        if g == 1:
            assert len(set(sizes)) == 1, sizes
            flat = sizes[0]
        else:
            assert max(sizes) <= flat and all(b <= a for a, b in zip(sizes, sizes[1:])), sizes
    fw = [ws(lib, 1, B=1, H=8, L=n, d=64, M=64, num_chunks=n // 512, window_chunks=64, group_slices=1)
          for n in (1 << 15, 1 << 20)]
    assert fw[0] == fw[1]


def test_state_handoff_sizes_and_checks(lib):
    # one window holds every slice: the states buffer holds (slices + 1) states of
    # (d + 1) x M fp32 per head, and a call given it needs that much less workspace
    d = d_(B=4, H=16, L=16384, d=64, M=256, num_chunks=32)
    slot = 65 * 256 * 4
    assert lib.slim_group_slices(ctypes.byref(d)) == 4  # 8 groups of four slices of 512
    assert lib.slim_state_bytes(ctypes.byref(d)) == 64 * 9 * slot
    d1 = d_(B=4, H=16, L=16384, d=64, M=256, num_chunks=32, group_slices=1)
    assert lib.slim_state_bytes(ctypes.byref(d1)) == 64 * 33 * slot
    for dd, n in ((d, 9), (d1, 33)):
        for p in (_lib.SLIM_PASS_FWD, _lib.SLIM_PASS_BWD):
            full = lib.slim_workspace_bytes(ctypes.byref(dd), p)
            assert 0 < lib.slim_workspace_bytes_states(ctypes.byref(dd), p) <= full - 64 * n * slot
    # a ragged last slice counts as a slice: L = 1000 in slices of 334 -> 3 slices, and
    # in groups of two: 2 groups (668 rows, then 332)
    dr = d_(B=1, H=2, L=1000, d=64, M=128, num_chunks=3)
    assert lib.slim_group_slices(ctypes.byref(dr)) == 1
    assert lib.slim_state_bytes(ctypes.byref(dr)) == 2 * 4 * 65 * 128 * 4
    dr2 = d_(B=1, H=2, L=1000, d=64, M=128, num_chunks=3, group_slices=2)
    assert lib.slim_state_bytes(ctypes.byref(dr2)) == 2 * 3 * 65 * 128 * 4
    # several windows: no states, and the workspace is the usual one
    dm = d_(B=1, H=8, L=1 << 20, d=64, M=64, num_chunks=2048, window_chunks=512)
    assert lib.slim_state_bytes(ctypes.byref(dm)) == 0
    for p in (_lib.SLIM_PASS_FWD, _lib.SLIM_PASS_BWD):
        assert lib.slim_workspace_bytes_states(ctypes.byref(dm), p) == lib.slim_workspace_bytes(ctypes.byref(dm), p)
    # the forward rejects states it cannot fill, and a workspace sized without them is
    # too small when no states are given; both before anything is enqueued
    assert fwd(lib, dm, states=P) == 2
    small = lib.slim_workspace_bytes_states(ctypes.byref(d), _lib.SLIM_PASS_FWD)
    assert fwd(lib, d, ws_bytes=small) == 5
    assert bwd(lib, d, ws_bytes=lib.slim_workspace_bytes_states(ctypes.byref(d), _lib.SLIM_PASS_BWD)) == 5
    assert fwd(lib, d, states=ctypes.c_void_p((1 << 20) + 4)) == 6
    assert bwd(lib, d, states=ctypes.c_void_p((1 << 20) + 4)) == 6
    assert lib.slim_state_bytes(ctypes.byref(d_(B=0))) == 0
    assert lib.slim_workspace_bytes_states(ctypes.byref(d_(B=0)), _lib.SLIM_PASS_FWD) == 0


def test_auto_window(lib):
    d = d_(B=4, H=16, L=16384, d=64, M=256, num_chunks=32)
    assert lib.slim_window_chunks(ctypes.byref(d)) == 32
    # the 1M-token workload fits one window within the 1 GiB budget of per-slice buffers
    d = d_(B=1, H=8, L=1 << 20, d=64, M=64, num_chunks=2048)
    assert lib.slim_window_chunks(ctypes.byref(d)) == 2048
    # a sequence whose per-slice buffers (slot, gradient slot, row statistics: 41 KB per
    # slice and head here) exceed 1 GiB gets windows of about 4096 workgroups again
    per = 8 * (65 * 64 * 4 * 2 + 512 * 16)
    assert 2048 * per <= 1 << 30 < 4096 * per
    d = d_(B=1, H=8, L=1 << 22, d=64, M=64, num_chunks=1 << 13, group_slices=1)
    assert lib.slim_window_chunks(ctypes.byref(d)) == 512
    # in groups of four slices (the automatic choice there): 512 workgroups of four slices
    d = d_(B=1, H=8, L=1 << 22, d=64, M=64, num_chunks=1 << 13)
    assert lib.slim_group_slices(ctypes.byref(d)) == 4
    assert lib.slim_window_chunks(ctypes.byref(d)) == 2048
    # many heads: about 4096 workgroups per launch when that is more; one group of
    # slices each (slices of 64 rows go 32 to a group)
    d = d_(B=64, H=64, L=4096, d=64, M=256, num_chunks=64, group_slices=1)
    assert lib.slim_window_chunks(ctypes.byref(d)) == 1
    d = d_(B=64, H=64, L=4096, d=64, M=256, num_chunks=64)
    assert lib.slim_group_slices(ctypes.byref(d)) == 32
    assert lib.slim_window_chunks(ctypes.byref(d)) == 32


def test_group_slices(lib):
    def g(**kw):
        return lib.slim_group_slices(ctypes.byref(d_(**kw)))
    # the largest power of two with groups of at most 2048 rows whose launches fill whole
    # rounds of each kernel's resident workgroups (512 for two 4-wave workgroups per CU,
    # 256 for the 8-wave dQ kernel at M = 256, 768 for three dQ workgroups at bf16 M = 64)
    # to within 10%
    assert g(B=4, H=16, L=16384, d=64, M=256, num_chunks=32) == 4        # 8 x 64 = 512: one round
    assert g(B=1, H=8, L=1 << 20, d=64, M=64, num_chunks=2048) == 2      # at 4, 4096 = 5.3 rounds of 768
    assert g(B=8, H=12, L=8192, d=128, M=128, num_chunks=32, feat=_lib.SLIM_FEAT_ELU1) == 2  # 4: 768 = 1.5 x 512
    assert g(B=2, H=8, L=4096, d=64, M=128, num_chunks=16) == 1          # 256 workgroups, not a round
    assert g(B=1, H=8, L=1 << 20, d=64, M=64, num_chunks=8192) == 8      # slices of 128: groups of 1024 rows
    assert g(B=64, H=64, L=4096, d=64, M=64, num_chunks=4) == 2          # slices of 1024 rows, 8192 workgroups
    assert g(B=64, H=16, L=1024, d=64, M=64, num_chunks=8) == 1          # 1024 at 8: 1.3 rounds of 768
    # given: taken as is, at most the slices there are
    assert g(group_slices=3) == 3
    assert g(L=1000, num_chunks=3, group_slices=5) == 3
    assert validate(lib, group_slices=-1) == 2
    # a window given in slices holds whole groups, at least one
    assert lib.slim_window_chunks(ctypes.byref(d_(L=4096, num_chunks=16, window_chunks=5, group_slices=2))) == 4
    assert lib.slim_window_chunks(ctypes.byref(d_(L=4096, num_chunks=16, window_chunks=1, group_slices=4))) == 4


def test_group_slices_invariants(lib):
    # over a grid of shapes: G is a power of two (or all the slices), at most 2048 rows per
    # group, and G > 1 only with at least one workgroup per CU (256; 512 where two
    # 4-wave workgroups share a CU: bf16 at d = 64, M = 256); the group count and the
    # states buffer follow from it
    for dtype in (_lib.SLIM_BF16, _lib.SLIM_F32):
        for B, H in ((1, 1), (1, 8), (4, 16), (8, 12), (64, 64)):
            for L, C in ((300, 3), (4096, 16), (16384, 32), (1 << 20, 2048), (1 << 20, 8192)):
                for d, M in ((64, 64), (64, 256), (128, 128)):
                    if B * H * L > (1 << 24):
                        continue
                    dd = d_(B=B, H=H, L=L, d=d, M=M, num_chunks=C, dtype=dtype)
                    G = lib.slim_group_slices(ctypes.byref(dd))
                    c = -(-L // C)
                    n = -(-L // c)
                    assert 1 <= G <= n and (G & (G - 1)) == 0, (B, H, L, C, d, M, G)
                    if G > 1:
                        least = 512 if (dtype == _lib.SLIM_BF16 and d == 64 and M == 256) else 256
                        assert G * c <= 2048 and -(-n // G) * B * H >= least, (B, H, L, C, d, M, G)
                    groups = -(-L // min(G * c, L))
                    if lib.slim_window_chunks(ctypes.byref(dd)) >= n:  # one window: states kept
                        assert lib.slim_state_bytes(ctypes.byref(dd)) == B * H * (groups + 1) * (d + 1) * M * 4


def test_tile_rows(lib):
    def tr(**kw):
        return lib.slim_tile_rows(ctypes.byref(d_(**kw)))
    assert tr(d=64, M=256) == 32                                   # bf16 FAVOR+ d=64 M=256
    # bf16 elu+1 at d = M = 128: 32-row tiles would take more than 80 KB of LDS in the
    # dK/dV kernel, so two workgroups could not share a compute unit
    assert tr(d=128, M=128, feat=_lib.SLIM_FEAT_ELU1) == 16
    assert tr(d=128, M=128, feat=_lib.SLIM_FEAT_ELU1, dtype=_lib.SLIM_F32) == 32
    assert tr(d=64, M=256, dtype=_lib.SLIM_F32) == 32
    assert tr(d=128, M=256) == 16                                  # 8 waves of d+4 fp32 reduction rows
    assert tr(d=128, M=256, dtype=_lib.SLIM_F32) == 16
    assert tr(d=16, M=16, dtype=_lib.SLIM_F32) == 32
    assert tr(d=48) == 0                                           # invalid descriptor


def test_decode_validation(lib):
    assert validate(lib, _lib.SLIM_PASS_DECODE, L=1, num_chunks=1) == 0
    assert validate(lib, _lib.SLIM_PASS_DECODE, L=2, num_chunks=1) == 2       # one token per head
    assert validate(lib, _lib.SLIM_PASS_DECODE, L=1, num_chunks=1, B=1 << 12, H=1 << 12) == 0
    assert validate(lib, _lib.SLIM_PASS_DECODE, L=1, num_chunks=1, B=1 << 12, H=(1 << 12) + 1) == 4
    assert validate(lib, 5) == 2                                              # unknown pass
    assert ws(lib, _lib.SLIM_PASS_DECODE, L=1, num_chunks=1) == 0


def test_decode_rejects_before_any_launch(lib):
    d = d_(L=1, num_chunks=1)
    p = ctypes.c_void_p(1 << 20)  # never dereferenced: every case fails on the host
    assert lib.slim_decode_step(ctypes.byref(d), None, p, p, p, None, None, p, p, p, None) == 1
    assert lib.slim_decode_step(ctypes.byref(d), p, p, p, None, None, None, p, p, p, None) == 1   # FAVOR+ W
    assert lib.slim_decode_step(ctypes.byref(d), p, p, p, p, p, None, p, p, p, None) == 1         # lone R_in
    assert lib.slim_decode_step(ctypes.byref(d), p, p, p, p, None, None, p, None, p, None) == 1   # R_out
    assert lib.slim_decode_step(ctypes.byref(d_(L=2, num_chunks=1)), p, p, p, p, None, None, p, p, p, None) == 2
    bad = ctypes.c_void_p((1 << 20) + 8)
    assert lib.slim_decode_step(ctypes.byref(d), p, p, p, p, None, None, bad, p, p, None) == 6
    # in place is allowed; a partly overlapping state is not
    r_in = ctypes.c_void_p(1 << 24)
    r_out = ctypes.c_void_p((1 << 24) + 256)
    s_ = ctypes.c_void_p(1 << 28)
    assert lib.slim_decode_step(ctypes.byref(d), p, p, p, p, r_in, s_, p, r_out, s_, None) == 2
    # with an fp64 state the ranges are twice as long: one state's length in fp32 bytes apart overlaps
    d64 = d_(L=1, num_chunks=1, state_dtype=_lib.SLIM_F64)
    r_far = ctypes.c_void_p((1 << 24) + 2 * 3 * 64 * 128 * 4)
    assert lib.slim_decode_step(ctypes.byref(d64), p, p, p, p, r_in, s_, p, r_far, s_, None) == 2
    de = d_(L=1, num_chunks=1, feat=_lib.SLIM_FEAT_ELU1, M=64)
    assert lib.slim_decode_step(ctypes.byref(de), p, p, p, p, None, None, p, p, p, None) == 2    # elu+1: no W


def test_state_dtype_validation(lib):
    assert validate(lib, _lib.SLIM_PASS_FWD, state_dtype=_lib.SLIM_F64) == 0
    assert validate(lib, _lib.SLIM_PASS_BWD, state_dtype=_lib.SLIM_F64) == 0
    assert validate(lib, _lib.SLIM_PASS_FWD, state_dtype=_lib.SLIM_BF16) == 3     # states are fp32 or fp64
    assert validate(lib, _lib.SLIM_PASS_FWD, state_dtype=7) == 3
    assert validate(lib, _lib.SLIM_PASS_DECODE, L=1, num_chunks=1, state_dtype=_lib.SLIM_F64) == 0  # fp64 state
    # the workspace does not depend on the state type (the carries are fp64 either way)
    assert ws(lib, 2, state_dtype=_lib.SLIM_F64) == ws(lib, 2)


def test_noalloc_forward_rejects_before_any_launch(lib):
    # the allocation-free forward checks its arguments and the fit of its workspace in
    # the fixed scratch array on the host, before any HIP call
    args = [P] * 3 + [P, None, None, P, P, P, None, None, None]  # Q K V W R_in S_in Y R_out S_out koff rs stream
    assert lib.slim_attn_fwd_noalloc(None, *args) == 1
    assert lib.slim_attn_fwd_noalloc(ctypes.byref(d_(num_chunks=0)), *args) == 2
    null_q = [None] + args[1:]
    assert lib.slim_attn_fwd_noalloc(ctypes.byref(d_()), *null_q) == 1
    bad = ctypes.c_void_p((1 << 20) + 4)
    assert lib.slim_attn_fwd_noalloc(ctypes.byref(d_()), bad, *args[1:]) == 6
    # two state slots and the fp64 carries of 600 heads at d = 64, M = 256 exceed 64 MiB
    too_many = d_(B=600, H=1, L=16, d=64, M=256, num_chunks=1)
    assert lib.slim_attn_fwd_noalloc(ctypes.byref(too_many), *args) == 5
    # an explicit window that does not fit is refused, not shrunk (one slice per
    # workgroup: 33 slots per head)
    wide = d_(B=64, H=1, L=16384, d=64, M=256, num_chunks=32, window_chunks=32, group_slices=1)
    assert lib.slim_attn_fwd_noalloc(ctypes.byref(wide), *args) == 5
    assert _lib.SLIM_NOALLOC_SCRATCH_BYTES == 64 << 20
