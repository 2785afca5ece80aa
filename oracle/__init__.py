"""CPU oracle of CoWindow Attention — test infrastructure, never part of the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import this package.  It shares no code with the GPU library.
"""

from .cowa_oracle import (  # noqa: F401
    COMPLEMENTARY, DENSE, DUPLICATED, MODES, Window, attn_bwd, attn_bwd_dkdv_cols,
    attn_bwd_dq_rows, attn_fwd, complementary_width, decode, default_scale, edge_counts,
    full_mask, mala_bwd, mala_bwd_dkdv_cols, mala_bwd_dq_rows, mala_fwd, mala_tile_mass, mask_rows,
    tile_lists,
)
