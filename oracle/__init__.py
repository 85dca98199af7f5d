"""CPU oracle for the TwELL sparse gated-FFN forward — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The product path (the HIP library and its Python binding) never
imports, links or calls anything here, and this package never imports the
product path. It shares no code with it.

Parity status: every function below is pinned by `-m "not gpu"` tests in
tests/test_oracle.py (closed forms, exact-integer brute force, a library
routine for the packing, invariants, degenerate densities). No function is
"parity unpinned"; absolute output values are pinned by the definition only,
since the pages print no worked numeric example.
"""

from .twell_oracle import (  # noqa: F401
    HybridFormat,
    TwellPacking,
    column_activity,
    column_rms,
    compact_rows,
    decode_bf16,
    dense_gated_ffn,
    ffn_from_active_set,
    ffn_backward,
    ffn_backward_from_hybrid,
    ffn_from_hidden_packing,
    ffn_from_twell,
    gate_preactivations,
    hybrid_pack,
    live_layout,
    overflow_rows,
    pack_twell,
    pack_twell_hidden,
    unpack_twell,
    up_projections,
)
