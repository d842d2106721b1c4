"""Unified paged, variable-length attention for MI355X (gfx950).

The computation lives in hand-written HIP kernels behind a C ABI
(``include/ua.h``, built as ``libua.so``); this package is the thin Python
binding over it.
"""

from .binding import (UA_BF16, UA_F16, UA_FP8_E4M3FN, UA_PATH_2D, UA_PATH_AUTO,  # noqa: F401
                      UA_PATH_SPLITKV, UaArgs, UaError, UaPlan, UaProblem, lib, ua_abi_version,
                      ua_forward_2d, ua_forward_noalloc, ua_forward_splitkv, ua_plan,
                      ua_reduce, ua_workspace_acc_offset)


def forward(*args, **kwargs):
    """See :func:`paged_varlen_attention_ua_amd.attention.forward`."""
    from .attention import forward as _fwd
    return _fwd(*args, **kwargs)
