"""MI355X-native causal linear self-attention (SLiM chunked prefix-sum scheme).

The computation lives in libslim.so (HIP, gfx950) behind the C ABI declared in
include/slim.h; this package is its thin Python binding.  Importing the
package does not load the library; the first call does, and fails loudly if
the library has not been built.
"""
from . import _lib  # noqa: F401

__all__ = ["featmap", "attn_fwd", "attn_bwd", "slim_attention", "decode_step"]


def __getattr__(name):
    if name in __all__:
        from . import attention
        return getattr(attention, name)
    raise AttributeError(name)
