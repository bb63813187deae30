"""Packed-bitmask apply for AMD Instinct MI355X (gfx950).

Applies a packed int32 allow-mask to [batch, vocab] logits: token v of row b
is kept when bit v % 32 of word mask[b, v // 32] is set, otherwise it is
replaced by -inf (in place) or by a caller-given fill value (out of place),
honouring the vocab-size/padding rule and an optional row-index list
(XGrammar "Bitmask Operations"; Modular MAX "apply_packed_bitmask").

The work is done by hand-written HIP kernels behind a C ABI
(include/mi_bitmask.h, libmi_bitmask.so); this package only marshals
arguments.  It raises ImportError-style errors if the library was not built.
"""

from ._binding import (  # noqa: F401
    BitmaskError,
    EXPORTS,
    MI_DTYPE,
    VARIANT,
    fill_value_bits,
    host_isa,
    load_library,
    mi_apply_bitmask_inplace,
    mi_apply_bitmask_inplace_host,
    mi_apply_bitmask_out,
    mi_apply_bitmask_out_host,
    mi_apply_bitmask_rows,
    mi_apply_bitmask_sample,
    mi_apply_bitmask_sample_noalloc,
    resolve_vocab_size,
    sample_workspace_bytes,
)
from .staging import MaskStager  # noqa: F401
from .xgrammar_api import (  # noqa: F401
    allocate_token_bitmask,
    apply_token_bitmask_inplace,
    bitmask_dtype,
    get_bitmask_shape,
    reset_token_bitmask,
)

__all__ = [
    "BitmaskError", "EXPORTS", "MI_DTYPE", "VARIANT", "fill_value_bits", "host_isa", "load_library",
    "mi_apply_bitmask_inplace", "mi_apply_bitmask_out", "mi_apply_bitmask_inplace_host",
    "mi_apply_bitmask_out_host", "mi_apply_bitmask_rows", "mi_apply_bitmask_sample", "mi_apply_bitmask_sample_noalloc",
    "resolve_vocab_size",
    "sample_workspace_bytes",
    "allocate_token_bitmask", "apply_token_bitmask_inplace", "bitmask_dtype", "get_bitmask_shape",
    "reset_token_bitmask", "MaskStager",
]
