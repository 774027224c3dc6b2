"""1.5-entmax (AdaSplash-style) attention on MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``libentmax_attn.so`` (``include/entmax_attn.h``); this package is the thin
Python binding plus the seeded input generators.  Build with
``__graft_entry__.build()`` (or ``python -m entmax_amd.build``).
"""

from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    EntmaxError,
    bwd_workspace_bytes,
    decode_bwd_workspace_bytes,
    decode_workspace_bytes,
    entmax_attn_bwd,
    entmax_attn_bwd_noalloc,
    entmax_attn_bwd_saved,
    entmax_attn_decode,
    entmax_attn_decode_bwd,
    entmax_attn_fwd,
    entmax_attn_fwd_save,
    entmax_attn_probs,
    entmax15_rows,
    entmax15_rows_bwd,
    entmax_bisect_rows,
    entmax_bisect_rows_bwd,
    load_library,
    saved_bytes,
)
