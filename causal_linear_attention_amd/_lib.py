"""ctypes binding of libslim.so (include/slim.h).  Argument marshalling only.

Loading fails loudly: there is no fallback implementation.  Build the library
with ``python -m causal_linear_attention_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libslim.so")

SLIM_F32, SLIM_BF16, SLIM_F64 = 0, 1, 2
SLIM_FEAT_FAVOR, SLIM_FEAT_ELU1 = 0, 1
SLIM_PASS_FEATMAP, SLIM_PASS_FWD, SLIM_PASS_BWD, SLIM_PASS_DECODE, SLIM_PASS_BWD_DW = 0, 1, 2, 3, 4
SLIM_NOALLOC_SCRATCH_BYTES = 64 << 20
STATUS = {0: "SLIM_OK", 1: "SLIM_ERR_NULL", 2: "SLIM_ERR_SHAPE", 3: "SLIM_ERR_DTYPE",
          4: "SLIM_ERR_UNSUPPORTED", 5: "SLIM_ERR_WORKSPACE", 6: "SLIM_ERR_ALIGN", 7: "SLIM_ERR_HIP"}

# every symbol declared in include/slim.h
EXPORTS = ["slim_validate", "slim_workspace_bytes", "slim_workspace_bytes_states", "slim_state_bytes",
           "slim_window_chunks", "slim_group_slices", "slim_tile_rows", "slim_featmap", "slim_attn_fwd", "slim_attn_fwd_noalloc",
           "slim_attn_bwd", "slim_decode_step", "slim_status_string", "slim_version", "slim_prof_enable",
           "slim_prof_count", "slim_prof_entry"]


class SlimDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("L", ctypes.c_int64), ("d", ctypes.c_int64),
                ("M", ctypes.c_int64), ("num_chunks", ctypes.c_int64), ("window_chunks", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("feat", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
                ("group_slices", ctypes.c_int32)]


class SlimError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({status_string(code)})")


_lib = None


def lib(path: str | None = None):
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libslim.so not found at {p}: build it with "
                           "`python -m causal_linear_attention_amd.build` (no CPU fallback exists)")
    L = ctypes.CDLL(p)
    vp, i32, sz, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int64
    D = ctypes.POINTER(SlimDesc)
    L.slim_validate.argtypes = [D, i32]
    L.slim_validate.restype = i32
    L.slim_workspace_bytes.argtypes = [D, i32]
    L.slim_workspace_bytes.restype = sz
    L.slim_workspace_bytes_states.argtypes = [D, i32]
    L.slim_workspace_bytes_states.restype = sz
    L.slim_state_bytes.argtypes = [D]
    L.slim_state_bytes.restype = sz
    L.slim_window_chunks.argtypes = [D]
    L.slim_window_chunks.restype = i64
    L.slim_group_slices.argtypes = [D]
    L.slim_group_slices.restype = i64
    L.slim_tile_rows.argtypes = [D]
    L.slim_tile_rows.restype = i64
    L.slim_featmap.argtypes = [D, vp, vp, vp, vp, vp]
    L.slim_featmap.restype = i32
    L.slim_attn_fwd.argtypes = [D] + [vp] * 13 + [sz, vp]
    L.slim_attn_fwd.restype = i32
    L.slim_attn_fwd_noalloc.argtypes = [D] + [vp] * 12
    L.slim_attn_fwd_noalloc.restype = i32
    L.slim_attn_bwd.argtypes = [D] + [vp] * 19 + [sz, vp]
    L.slim_attn_bwd.restype = i32
    L.slim_decode_step.argtypes = [D, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.slim_decode_step.restype = i32
    L.slim_status_string.argtypes = [i32]
    L.slim_status_string.restype = ctypes.c_char_p
    L.slim_version.argtypes = []
    L.slim_version.restype = i32
    L.slim_prof_enable.argtypes = [i32]
    L.slim_prof_enable.restype = i32
    L.slim_prof_count.argtypes = []
    L.slim_prof_count.restype = i32
    L.slim_prof_entry.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(ctypes.c_int64)]
    L.slim_prof_entry.restype = i32
    if path is None:
        _lib = L
    return L


def status_string(code: int) -> str:
    try:
        return lib().slim_status_string(int(code)).decode()
    except Exception:  # noqa: BLE001 - used while formatting another error
        return "?"


def check(code: int, where: str):
    if code != 0:
        raise SlimError(code, where)


def desc(B, H, L, d, M, num_chunks=1, window_chunks=0, dtype=SLIM_F32, feat=SLIM_FEAT_FAVOR,
         state_dtype=SLIM_F32, group_slices=0) -> SlimDesc:
    return SlimDesc(int(B), int(H), int(L), int(d), int(M), int(num_chunks), int(window_chunks), int(dtype),
                    int(feat), int(state_dtype), int(group_slices))


def prof_enable(on: bool):
    check(lib().slim_prof_enable(1 if on else 0), "slim_prof_enable")


def prof_read() -> dict:
    """{kernel name: (total GPU ms, launches)} since the last prof_enable(True)."""
    L = lib()
    out = {}
    for i in range(L.slim_prof_count()):
        name, ms, n = ctypes.c_char_p(), ctypes.c_double(), ctypes.c_int64()
        check(L.slim_prof_entry(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n)), "slim_prof_entry")
        out[name.value.decode()] = (ms.value, n.value)
    return out
