"""Structured-mask softmax attention for AMD MI355X (gfx950).

The compute path is the HIP library ``libbss_attn.so`` built from ``csrc/``
(C ABI in ``include/bss_attn.h``); this package only marshals arguments.
"""

from ._lib import (  # noqa: F401
    AttnError,
    Plan,
    PreparedBackward,
    PreparedDecode,
    PreparedMask,
    RrSearch,
    bind_group,
    decode_fwd,
    load_library,
    masked_bwd,
    masked_fwd,
    masked_fwd_lse,
    masked_fwd_oneshot,
    prepare,
    prepare_backward,
    reorder_tokens,
    rr_search,
    tensor_view,
)

__all__ = ["AttnError", "Plan", "PreparedBackward", "PreparedDecode", "decode_fwd", "PreparedMask", "RrSearch", "bind_group", "load_library",
           "masked_bwd", "masked_fwd", "masked_fwd_lse", "masked_fwd_oneshot", "prepare", "prepare_backward",
           "reorder_tokens", "rr_search", "tensor_view"]
