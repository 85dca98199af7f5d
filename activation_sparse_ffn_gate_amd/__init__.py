"""TwELL sparse gated-FFN forward on MI355X (gfx950).

The computation lives in libtwell.so (hand-written HIP kernels behind the C ABI
declared in include/twell.h). This package is its thin Python binding: it
passes device pointers of torch tensors and the current stream, nothing more.
"""

from ._lib import (  # noqa: F401
    OP_COLUMN_ACTIVITY,
    OP_DENSE_FALLBACK,
    OP_DENSE_FFN,
    OP_FFN_FORWARD,
    OP_FFN_FORWARD_GATEUP,
    OP_GATE_PACK,
    OP_SLICED_UPDOWN,
    LIB_PATH,
    Hybrid,
    Packed,
    Spill,
    TwellError,
    Workspace,
    column_activity,
    compact_layer,
    backward_workspace_bytes,
    ctrl_bytes,
    dense_fallback,
    dense_ffn_forward,
    ffn_backward,
    ffn_forward,
    ffn_forward_static,
    ffn_forward_timed,
    ffn_forward_gateup,
    fused_updown,
    gate_pack,
    gate_pack_spill,
    gateup_pack,
    gather_rows,
    header_functions,
    hidden_down,
    hybrid_pack,
    lib,
    live_layout,
    packed_view,
    sliced_updown,
    status_string,
    workspace_bytes,
)
